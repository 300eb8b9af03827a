// Skinny MFMA GEMMs for batches between a decode step and a prompt chunk
// (an MTP verify batch of many sequences, 16 < T < 1,024 tokens), and the
// router of such batches.
//
// At these sizes an expert has a few to a few dozen rows, and a tile loop that
// walks K = 2,560 serially is bound by memory latency, not by the matrix
// cores.  Here a block takes one "chunk" (up to 32 rows of one expert group)
// and 64 output columns, and its W waves split K: wave w owns K steps
// [w UPW, (w + 1) UPW) of 64.  Every wave loads its A and B fragments straight
// from memory into registers (B dequantised there, mfma.h), two steps ahead of
// their use, runs 2 MFMA 32x32x16 per 16 K, and the W partial tiles are summed
// in LDS in wave order (deterministic) before the epilogue:
//   GateUp: h = SiLU(gate) * up for 32 gate + the 32 matching up columns,
//           fp16, pair order (the down projection's A operand);
//   Down:   64 output columns of y, fp32 (combined like the GEMV's rows);
//   Router: 64 experts' logits (+ bias), bf16 operands in natural order.
// Blocks walk the (chunk, column tile) space grid-stride, column tile fastest.
#include <math.h>

#include <algorithm>

#include "device.h"
#include "internal.h"
#include "mfma.h"

namespace moe {

enum class Skinny { GateUp, Down, Router };

struct SkinnyArgs {
  const uint8_t* r_codes;
  const uint16_t* r_scales;
  const uint8_t* s_codes;
  const uint16_t* s_scales;
  size_t code_stride, scale_stride;
  int H, I, E, T, k;
  const int32_t* tiles;      // chunks: (group, first sorted position, rows <= 32)
  const int32_t* n_tiles;
  const int32_t* sorted_rows;
  const uint16_t* a_src;     // GateUp: x fp16 pair order; Down: h fp16 pair order; Router: x bf16
  const uint16_t* wr;        // Router: bf16 [E][H]
  const float* bias;         // Router: fp32 [E] or NULL
  uint16_t* h_out;
  float* y_out;
  float* logits;
};

template <Skinny KIND, int W, int UPW>
__global__ __launch_bounds__(W * 64) void k_gemm_skinny(SkinnyArgs a) {
  constexpr bool ROUTER = KIND == Skinny::Router;
  __shared__ float red[W][16][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = KIND == Skinny::Down ? a.I : a.H;
  const int nch = K / 64;
  const int ncol = KIND == Skinny::GateUp ? a.I / 32 : (ROUTER ? (a.E + 63) / 64 : a.H / 64);
  const int nchunks = ROUTER ? (a.T + 31) / 32 : __builtin_amdgcn_readfirstlane(a.n_tiles[0]);
  const int units = nchunks * ncol;
  const int r32 = lane & 31, kh = (lane >> 5) * 8, shift = (lane >> 5) * 8;
  const BConst bc = bconst();

  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int chunk = unit / ncol, j = unit - chunk * ncol;
    int g = 0, m0, rows;
    if (ROUTER) {
      m0 = chunk * 32;
      rows = min(32, a.T - m0);
    } else {
      g = a.tiles[3 * chunk];
      m0 = a.tiles[3 * chunk + 1];
      rows = a.tiles[3 * chunk + 2];
    }
    // A row of this lane (rows past the chunk repeat its first row)
    const int rr = r32 < rows ? r32 : 0;
    size_t arow;
    if (KIND == Skinny::GateUp) {
      const int r = a.sorted_rows[m0 + rr];
      const int Tk = a.T * a.k;
      arow = (size_t)(r < Tk ? r / a.k : r - Tk);
    } else {
      arow = (size_t)(m0 + rr);
    }
    const u32x4* __restrict__ ap = reinterpret_cast<const u32x4*>(a.a_src + arow * K + kh);
    // B columns
    int n0, n1;
    if (KIND == Skinny::GateUp) {
      n0 = 32 * j + r32;
      n1 = a.I + n0;
    } else {
      n0 = 64 * j + r32;
      n1 = n0 + 32;
    }
    BCol B0, B1;
    const u32x4* __restrict__ w0 = nullptr;
    const u32x4* __restrict__ w1 = nullptr;
    if (ROUTER) {
      w0 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(n0, a.E - 1) * K + kh);
      w1 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(n1, a.E - 1) * K + kh);
    } else {
      const bool sh = g == a.E;
      const size_t eidx = sh ? 0 : (size_t)g;
      const uint8_t* codes = (sh ? a.s_codes : a.r_codes) + eidx * a.code_stride;
      const uint16_t* scales = (sh ? a.s_scales : a.r_scales) + eidx * a.scale_stride;
      B0 = b_column(codes, scales, n0, K);
      B1 = b_column(codes, scales, n1, K);
    }

    f16x_t acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;

    // registers of the wave's UPW steps; loads issued two steps ahead of use
    u32x4 A[UPW][4];
    u32x4 WB[ROUTER ? UPW : 1][8];
    BRegs QB[ROUTER ? 1 : UPW];
    auto issue = [&](int u) {
      const int step = min(wv * UPW + u, nch - 1);   // past the end: reload the last step, result unused
#pragma unroll
      for (int s = 0; s < 4; ++s) A[u][s] = ap[step * 8 + 2 * s];
      if (ROUTER) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          WB[u][s] = w0[step * 8 + 2 * s];
          WB[u][4 + s] = w1[step * 8 + 2 * s];
        }
      } else {
        load_b(B0, B1, step, QB[u]);
      }
    };
    auto compute = [&](int u) {
      if (wv * UPW + u >= nch) return;   // wave-uniform
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (ROUTER) {
          const b8_t fa = __builtin_bit_cast(b8_t, A[u][s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, WB[u][s]), acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, WB[u][4 + s]), acc1, 0, 0, 0);
        } else {
          const uint32_t c0 = QB[u].c0[s], c1 = QB[u].c1[s];
          const h8_t b0 = b_frag(c0 >> shift, scale_pair(QB[u].s0, s >= 2), bc);
          const h8_t b1 = b_frag(c1 >> shift, scale_pair(QB[u].s1, s >= 2), bc);
          const h8_t fa = __builtin_bit_cast(h8_t, A[u][s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, b0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, b1, acc1, 0, 0, 0);
        }
      }
    };
#pragma unroll
    for (int u = 0; u < UPW + 2; ++u) {
      if (u < UPW) issue(u);
      __builtin_amdgcn_sched_barrier(0);
      if (u >= 2) compute(u - 2);
    }

    // fixed-order reduction over the waves, one fragment at a time
    constexpr int PER = (1024 + W * 64 - 1) / (W * 64);   // outputs per thread
    float v0[PER], v1[PER];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wv][r][lane] = f ? acc1[r] : acc0[r];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int e = threadIdx.x + q * W * 64;
        float sum = 0.0f;
        if (e < 1024)
          for (int w = 0; w < W; ++w) sum += red[w][e >> 6][e & 63];
        if (f)
          v1[q] = sum;
        else
          v0[q] = sum;
      }
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = threadIdx.x + q * W * 64;
      if (e >= 1024) continue;
      const int r = e >> 6, l = e & 63;
      const int row = acc_row(r, l), col = l & 31;
      if (row >= rows) continue;
      if (KIND == Skinny::GateUp) {
        const float gv = v0[q], uv = v1[q];
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        const int c = 32 * j + col;
        const int pc = (c & ~15) + pair_pos(c & 15);
        a.h_out[(size_t)(m0 + row) * a.I + pc] = __builtin_bit_cast(uint16_t, (_Float16)hv);
      } else if (KIND == Skinny::Down) {
        float* yr = a.y_out + (size_t)(m0 + row) * a.H + 64 * j + col;
        yr[0] = v0[q];
        yr[32] = v1[q];
      } else {
        const int e0 = 64 * j + col, e1 = e0 + 32;
        float* lr = a.logits + (size_t)(m0 + row) * a.E;
        if (e0 < a.E) lr[e0] = v0[q] + (a.bias ? a.bias[e0] : 0.0f);
        if (e1 < a.E) lr[e1] = v1[q] + (a.bias ? a.bias[e1] : 0.0f);
      }
    }
    __syncthreads();   // red is reused by the next unit
  }
}

static constexpr int kSkinnyWaves = 8;

template <Skinny KIND>
static hipError_t launch_skinny_t(const SkinnyArgs& a, int units, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  const int K = KIND == Skinny::Down ? a.I : a.H;
  const int nch = K / 64;
  dim3 grid(units), block(kSkinnyWaves * 64);
  if (nch <= 2 * kSkinnyWaves)
    MOE_LAUNCH((k_gemm_skinny<KIND, kSkinnyWaves, 2>), grid, block, 0, s, a);
  else if (nch <= 5 * kSkinnyWaves)
    MOE_LAUNCH((k_gemm_skinny<KIND, kSkinnyWaves, 5>), grid, block, 0, s, a);
  else if (nch <= 8 * kSkinnyWaves)
    MOE_LAUNCH((k_gemm_skinny<KIND, kSkinnyWaves, 8>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Grouped skinny GEMM over the chunks of a plan (32-row tiles of every group).
// max_chunks bounds the chunk count (known on the device only); the grid is at
// most a few blocks per CU and walks the units grid-stride.
hipError_t launch_gemm_skinny(GemvKind kind, const MatRef& routed, const MatRef& shared, int H, int I, int E,
                              const int32_t* chunks, const int32_t* n_chunks, int max_chunks,
                              const int32_t* sorted_rows, int T, int k, const uint16_t* a_f16, void* out,
                              hipStream_t s) {
  SkinnyArgs a = {};
  a.r_codes = routed.codes;
  a.r_scales = routed.scales;
  a.s_codes = shared.codes;
  a.s_scales = shared.scales;
  a.code_stride = routed.code_stride;
  a.scale_stride = routed.scale_stride;
  a.H = H;
  a.I = I;
  a.E = E;
  a.T = T;
  a.k = k;
  a.tiles = chunks;
  a.n_tiles = n_chunks;
  a.sorted_rows = sorted_rows;
  a.a_src = a_f16;
  const int cols = kind == GemvKind::GateUp ? I / 32 : H / 64;
  const int units = std::min(max_chunks * cols, 2048);
  if (kind == GemvKind::GateUp) {
    a.h_out = (uint16_t*)out;
    return launch_skinny_t<Skinny::GateUp>(a, units, s);
  }
  a.y_out = (float*)out;
  return launch_skinny_t<Skinny::Down>(a, units, s);
}

hipError_t launch_router_skinny(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                                float* logits, hipStream_t s) {
  SkinnyArgs a = {};
  a.H = H;
  a.E = E;
  a.T = T;
  a.a_src = x;
  a.wr = wr;
  a.bias = bias;
  a.logits = logits;
  const int units = ((T + 31) / 32) * ((E + 63) / 64);
  return launch_skinny_t<Skinny::Router>(a, units, s);
}

}  // namespace moe

// MFMA grouped GEMMs for prefill chunks and large token groups, and the MFMA
// router GEMM.
//
// A prompt is read in chunks of up to 8,192 tokens (page "Strata Runs a
// 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU at up to 93 Tokens per
// Second"); for such a chunk every expert that a few dozen or more tokens chose
// is a dense [M_e x 2560] x [2560 x 1280] product followed by [M_e x 640] x
// [640 x 2560], which belongs on the matrix cores.
//
// Precision: the weights are dequantised EXACTLY into fp16 (s * (c - 2) with an
// fp16 scale and c - 2 in {-2, -1, 0, 1} is an fp16 value), activations enter as
// fp16 (bf16 -> fp16 is exact for |x| >= 2^-17 and below 65504), products are
// exact and accumulate in fp32 (v_mfma_f32_32x32x16_f16); h = SiLU(gate) * up is
// carried in fp16 between the two GEMMs and the output is fp32.
//
// Operand order: the 2-bit unpacking yields weights in "pair order" -- inside
// each aligned group of 16 columns the order is (0, 8, 1, 9, ..., 7, 15).  The
// MFMA sums over K in any order as long as both operands agree, so the fp16
// activations (x, and h from the gate/up epilogue) are stored in the same order
// and no operand is ever permuted inside the GEMM.
//
// Tiles: a block computes 128 rows (sorted positions of one expert) x 128
// columns with 4 waves of 64 x 64 (2 x 2 MFMA 32x32 tiles); the K loop steps by
// 64 with double-buffered LDS: the next step's global loads are in flight while
// the current step's MFMAs run, and the dequantisation happens on the way into
// LDS.  The gate/up kernel's 128 columns are 64 gate + the 64 matching up
// columns, so SwiGLU is applied in registers.
#include <math.h>

#include "device.h"
#include "internal.h"

namespace moe {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int LDS_STRIDE = BK + 8;   // halves per LDS row (padding against bank conflicts)

// position of column k (0..15) of a 16-group in pair order
__device__ __forceinline__ int pair_pos(int k) { return k < 8 ? 2 * k : 2 * (k - 8) + 1; }

// ---------------------------------------------------------------------------
// x (bf16) -> fp16 in pair order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_x_to_f16_pairs(const uint16_t* __restrict__ x, size_t n16,
                                                        uint16_t* __restrict__ out) {
  // one thread per 16-group
  for (size_t g = (size_t)blockIdx.x * 256 + threadIdx.x; g < n16; g += (size_t)gridDim.x * 256) {
    const uint4* src = reinterpret_cast<const uint4*>(x + g * 16);
    const uint4 a = src[0], b = src[1];
    const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column j (low half of in[j/2] if j even) and column j + 8
      const uint32_t v0 = (j & 1) ? (in[j >> 1] >> 16) : (in[j >> 1] & 0xFFFFu);
      const uint32_t v1 = (j & 1) ? (in[4 + (j >> 1)] >> 16) : (in[4 + (j >> 1)] & 0xFFFFu);
      const _Float16 f0 = (_Float16)bf16_to_f32(v0), f1 = (_Float16)bf16_to_f32(v1);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, f0) | ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + g * 16);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

hipError_t launch_x_to_f16_pairs(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s) {
  const size_t n16 = (size_t)T * H / 16;
  const int blocks = (int)((n16 + 255) / 256 < 2048 ? (n16 + 255) / 256 : 2048);
  hipLaunchKernelGGL(k_x_to_f16_pairs, dim3(blocks), dim3(256), 0, s, x, n16, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exact fp16 dequantisation of one 2-bit word (16 weights) into 8 pair-order
// dwords: pair j = (w_j, w_{j+8}) as (fp16, fp16).  Codes at bits 0..9 of each
// half fit the fp16 significand under the exponent of 1024 (value 1024 + c 2^p);
// v_pk_fma_f16 turns that into c - 2 exactly and v_pk_mul_f16 applies the scale.
// ---------------------------------------------------------------------------
struct Dq16 {
  uint32_t mask[5];   // 0x00030003 << 2j, j = 0..4
  uint32_t magic;     // 0x64006400
  h2_t mul[5];        // 2^-p
  h2_t add[5];        // -(1024 * 2^-p + 2)
};

__device__ __forceinline__ Dq16 dq16_consts() {
  Dq16 d;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    d.mask[j] = vgpr_const(0x00030003u << (2 * j));
    const float m = ldexpf(1.0f, -2 * j);
    d.mul[j] = h2_t{(_Float16)m, (_Float16)m};
    d.add[j] = h2_t{(_Float16)(-(1024.0f * m + 2.0f)), (_Float16)(-(1024.0f * m + 2.0f))};
  }
  d.magic = vgpr_const(0x64006400u);
  return d;
}

__device__ __forceinline__ uint32_t dq_pair(uint32_t w, int j, const Dq16& d, h2_t s2) {
  // pairs 0..4 in place, 5..7 from w >> 10 at positions 0..2
  const int q = j < 5 ? j : j - 5;
  const uint32_t src = j < 5 ? w : (w >> 10);
  const uint32_t v = (src & d.mask[q]) | d.magic;
  h2_t f = __builtin_bit_cast(h2_t, v);
  f = f * d.mul[q] + d.add[q];      // exact: c - 2
  f = f * s2;                        // exact: s * (c - 2)
  return __builtin_bit_cast(uint32_t, f);
}

// ---------------------------------------------------------------------------
// MFMA fragments from LDS and the 2 x 2 wave tile
// ---------------------------------------------------------------------------
__device__ __forceinline__ h8_t lds_frag(const uint16_t* base, int row, int k) {
  return *reinterpret_cast<const h8_t*>(base + row * LDS_STRIDE + k);
}

// acc[mi][ni] += A[rows a0 + 32 mi ..][k] * B[cols b0 + 32 ni ..][k] over one BK step
__device__ __forceinline__ void wave_mfma_step(const uint16_t* As, const uint16_t* Bs, int a0, int b0_0, int b0_1,
                                               f16x_t acc[2][2]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int k16 = 0; k16 < BK; k16 += 16) {
    const h8_t fa0 = lds_frag(As, a0 + r, k16 + kh);
    const h8_t fa1 = lds_frag(As, a0 + 32 + r, k16 + kh);
    const h8_t fb0 = lds_frag(Bs, b0_0 + r, k16 + kh);
    const h8_t fb1 = lds_frag(Bs, b0_1 + r, k16 + kh);
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0, fb0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0, fb1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1, fb0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1, fb1, acc[1][1], 0, 0, 0);
  }
}

// row (0..31) of accumulator register r for this lane, column = lane & 31
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Global loads of one K step for one thread: 32 fp16 activations, 2 code words
// and the block's fp16 scale.
struct Prefetch {
  uint4 a[4];
  uint2 b;
  uint32_t s;
};

// Software pipeline over the K steps with two register sets: while the MFMAs of
// step kc run out of LDS buffer kc % 2, the loads of step kc + 2 are in flight
// and step kc + 1 (loaded one iteration earlier) is dequantised into the other
// buffer.  Unrolled by two so that both register sets have static names.
#define K_PIPELINE(MFMA_BUF0, MFMA_BUF1)                 \
  Prefetch P0, P1;                                       \
  load_step(P0, 0);                                      \
  if (nch > 1) load_step(P1, 1);                         \
  store_step(P0, 0);                                     \
  __syncthreads();                                       \
  for (int kc = 0; kc < nch; kc += 2) {                  \
    if (kc + 2 < nch) load_step(P0, kc + 2);             \
    MFMA_BUF0;                                           \
    if (kc + 1 < nch) store_step(P1, 1);                 \
    __syncthreads();                                     \
    if (kc + 1 >= nch) break;                            \
    if (kc + 3 < nch) load_step(P1, kc + 3);             \
    MFMA_BUF1;                                           \
    if (kc + 2 < nch) store_step(P0, 0);                 \
    __syncthreads();                                     \
  }

// ---------------------------------------------------------------------------
// Grouped GEMM tiles: (group, first sorted position, rows <= BM) per M-tile.
// ---------------------------------------------------------------------------
struct GemmTile {
  int g, m0, rows, n;   // n = column-tile index
};

// Workgroups are placed on the 8 XCDs round-robin by linear id.  Only the
// first n_valid = tiles x column-tiles linear ids carry work (the grid is a host
// bound); re-number those so that XCD x runs a contiguous range of logical
// tiles, column-tile fastest: the column tiles of one row tile then share its
// activation rows in one L2, and every XCD still gets 1/8 of the work.
__device__ __forceinline__ int xcd_logical_id(int lin, int n_valid) {
  const int per = (n_valid + 7) / 8;
  const int xcd = lin & 7, slot = lin >> 3;
  const int full = n_valid - 8 * (per - 1);   // XCDs that get `per` ids (the rest get per - 1)
  return xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
}

__device__ __forceinline__ bool load_tile(const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
                                          GemmTile& t) {
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int n_valid = n_tiles[0] * (int)gridDim.y;
  if (lin >= n_valid) return false;
  const int id = xcd_logical_id(lin, n_valid);
  const int mt = id / gridDim.y;
  t.n = id % gridDim.y;
  t.g = tiles[3 * mt];
  t.m0 = tiles[3 * mt + 1];
  t.rows = tiles[3 * mt + 2];
  return true;
}

// ---------------------------------------------------------------------------
// Gate/up: h[p, n] = SiLU(x_t . Wg[n]) * (x_t . Wu[n]) for the tile's rows p
// (token t of sorted position p), columns n in [64 * t.n, +64).
// LDS B rows 0..63 = gate rows, 64..127 = the matching up rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_gemm_gateup_q2(
    const uint8_t* __restrict__ r_codes, const uint16_t* __restrict__ r_scales, const uint8_t* __restrict__ s_codes,
    const uint16_t* __restrict__ s_scales, size_t code_stride, size_t scale_stride, int H, int I, int E,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ sorted_rows,
    int T, int k, const uint16_t* __restrict__ xh, uint16_t* __restrict__ h_out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  GemmTile t;
  if (!load_tile(tiles, n_tiles, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool sh = t.g == E;
  const size_t eidx = sh ? 0 : (size_t)t.g;
  const uint8_t* __restrict__ codes = (sh ? s_codes : r_codes) + eidx * code_stride;
  const uint16_t* __restrict__ scales = (sh ? s_scales : r_scales) + eidx * scale_stride;
  const int nch = H / 64, n128 = H / 128;

  // A: thread -> (row ra = tid / 2, half ha = tid % 2): 32 fp16 of the row per step
  const int ra = tid >> 1, ha = tid & 1;
  int tok;
  {
    const int p = t.m0 + (ra < t.rows ? ra : 0);
    const int r = sorted_rows[p];
    const int Tk = T * k;
    tok = r < Tk ? r / k : r - Tk;
  }
  const uint4* __restrict__ arow = reinterpret_cast<const uint4*>(xh + (size_t)tok * H) + ha * 4;
  // B: thread -> (LDS row rb = tid / 2: gate rows 0..63, up rows 64..127; half hb = block within the chunk)
  const int rb = tid >> 1, hb = tid & 1;
  const int wrow = (rb < 64) ? t.n * 64 + rb : I + t.n * 64 + (rb - 64);
  const int ng = wrow >> 6, rl = wrow & 63;
  const uint2* __restrict__ bcode = reinterpret_cast<const uint2*>(codes) + ((size_t)ng * nch * 64 + rl) * 2 + hb;
  const Dq16 D = dq16_consts();

  auto load_step = [&](Prefetch& P, int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) P.a[q] = arow[kc * 8 + q];
    P.b = bcode[(size_t)kc * 64 * 2];
    const int blk = 2 * kc + hb;
    P.s = scales[(((size_t)ng * n128 + (blk >> 2)) * 64 + rl) * 4 + (blk & 3)];
  };
  auto store_step = [&](const Prefetch& P, int buf) {
    uint16_t* a = &As[buf][ra * LDS_STRIDE + ha * 32];
#pragma unroll
    for (int q = 0; q < 4; ++q) reinterpret_cast<uint4*>(a)[q] = P.a[q];
    const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)P.s);
    const h2_t s2 = h2_t{sv, sv};
    uint32_t o[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o[j] = dq_pair(P.b.x, j, D, s2);
      o[8 + j] = dq_pair(P.b.y, j, D, s2);
    }
    uint4* b = reinterpret_cast<uint4*>(&Bs[buf][rb * LDS_STRIDE + hb * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  };

  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // wave tile: rows (wv >> 1) * 64, gate cols (wv & 1) * 32 and the matching up cols
  const int a0 = (wv >> 1) * 64;
  const int bg = (wv & 1) * 32, bu = 64 + (wv & 1) * 32;

  K_PIPELINE(wave_mfma_step(As[0], Bs[0], a0, bg, bu, acc), wave_mfma_step(As[1], Bs[1], a0, bg, bu, acc));
  // epilogue: SwiGLU in registers, h stored in pair order
  const int col = t.n * 64 + (wv & 1) * 32 + (lane & 31);
  const int pcol = (col & ~15) + pair_pos(col & 15);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = a0 + 32 * mi + acc_row(r, lane);
      if (row < t.rows) {
        const float g = acc[mi][0][r], u = acc[mi][1][r];
        const float hv = g / (1.0f + expf(-g)) * u;
        h_out[(size_t)(t.m0 + row) * I + pcol] = __builtin_bit_cast(uint16_t, (_Float16)hv);
      }
    }
}

// ---------------------------------------------------------------------------
// Down: y[p, n] = h[p] . Wd[n] for the tile's rows, n in [128 * t.n, +128).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_gemm_down_q2(
    const uint8_t* __restrict__ r_codes, const uint16_t* __restrict__ r_scales, const uint8_t* __restrict__ s_codes,
    const uint16_t* __restrict__ s_scales, size_t code_stride, size_t scale_stride, int H, int I, int E,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles, const uint16_t* __restrict__ hh,
    float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  GemmTile t;
  if (!load_tile(tiles, n_tiles, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool sh = t.g == E;
  const size_t eidx = sh ? 0 : (size_t)t.g;
  const uint8_t* __restrict__ codes = (sh ? s_codes : r_codes) + eidx * code_stride;
  const uint16_t* __restrict__ scales = (sh ? s_scales : r_scales) + eidx * scale_stride;
  const int nch = I / 64, n128 = I / 128;

  const int ra = tid >> 1, ha = tid & 1;
  const int prow = t.m0 + (ra < t.rows ? ra : 0);
  const uint4* __restrict__ arow = reinterpret_cast<const uint4*>(hh + (size_t)prow * I) + ha * 4;
  const int rb = tid >> 1, hb = tid & 1;
  const int wrow = t.n * 128 + rb;
  const int ng = wrow >> 6, rl = wrow & 63;
  const uint2* __restrict__ bcode = reinterpret_cast<const uint2*>(codes) + ((size_t)ng * nch * 64 + rl) * 2 + hb;
  const Dq16 D = dq16_consts();

  auto load_step = [&](Prefetch& P, int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) P.a[q] = arow[kc * 8 + q];
    P.b = bcode[(size_t)kc * 64 * 2];
    const int blk = 2 * kc + hb;
    P.s = scales[(((size_t)ng * n128 + (blk >> 2)) * 64 + rl) * 4 + (blk & 3)];
  };
  auto store_step = [&](const Prefetch& P, int buf) {
    uint16_t* a = &As[buf][ra * LDS_STRIDE + ha * 32];
#pragma unroll
    for (int q = 0; q < 4; ++q) reinterpret_cast<uint4*>(a)[q] = P.a[q];
    const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)P.s);
    const h2_t s2 = h2_t{sv, sv};
    uint32_t o[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o[j] = dq_pair(P.b.x, j, D, s2);
      o[8 + j] = dq_pair(P.b.y, j, D, s2);
    }
    uint4* b = reinterpret_cast<uint4*>(&Bs[buf][rb * LDS_STRIDE + hb * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  };

  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int a0 = (wv >> 1) * 64, b0 = (wv & 1) * 64;

  K_PIPELINE(wave_mfma_step(As[0], Bs[0], a0, b0, b0 + 32, acc), wave_mfma_step(As[1], Bs[1], a0, b0, b0 + 32, acc));
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = a0 + 32 * mi + acc_row(r, lane);
        if (row < t.rows) y[(size_t)(t.m0 + row) * H + t.n * 128 + b0 + 32 * ni + (lane & 31)] = acc[mi][ni][r];
      }
}

hipError_t launch_gemm_q2(GemvKind kind, const MatRef& routed, const MatRef& shared, int H, int I, int E,
                          const int32_t* tiles, const int32_t* n_tiles, int max_tiles, const int32_t* sorted_rows,
                          int T, int k, const uint16_t* a_f16, void* out, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (kind == GemvKind::GateUp) {
    hipLaunchKernelGGL(k_gemm_gateup_q2, dim3(max_tiles, I / 64), dim3(256), 0, s, routed.codes, routed.scales,
                       shared.codes, shared.scales, routed.code_stride, routed.scale_stride, H, I, E, tiles, n_tiles,
                       sorted_rows, T, k, a_f16, (uint16_t*)out);
  } else {
    hipLaunchKernelGGL(k_gemm_down_q2, dim3(max_tiles, H / 128), dim3(256), 0, s, routed.codes, routed.scales,
                       shared.codes, shared.scales, routed.code_stride, routed.scale_stride, H, I, E, tiles, n_tiles,
                       a_f16, (float*)out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router GEMM (bf16 MFMA): logits[t, e] = x_t . Wr[e] + b[e] for 128 x 128 tiles.
// Both operands are bf16 in natural column order; products are exact in fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ b8_t lds_frag_b(const uint16_t* base, int row, int k) {
  return *reinterpret_cast<const b8_t*>(base + row * LDS_STRIDE + k);
}

__global__ __launch_bounds__(256, 2) void k_router_mfma(const uint16_t* __restrict__ x, int T,
                                                        const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ bias, int E, int H,
                                                        float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int ra = tid >> 1, ha = tid & 1;
  const int arow_i = min(m0 + ra, T - 1), brow_i = min(n0 + ra, E - 1);
  const uint4* __restrict__ arow = reinterpret_cast<const uint4*>(x + (size_t)arow_i * H) + ha * 4;
  const uint4* __restrict__ brow = reinterpret_cast<const uint4*>(wr + (size_t)brow_i * H) + ha * 4;
  const int nch = H / 64;
  uint4 pa[4], pb[4];
  auto load_step = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa[q] = arow[kc * 8 + q];
      pb[q] = brow[kc * 8 + q];
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      reinterpret_cast<uint4*>(&As[buf][ra * LDS_STRIDE + ha * 32])[q] = pa[q];
      reinterpret_cast<uint4*>(&Bs[buf][ra * LDS_STRIDE + ha * 32])[q] = pb[q];
    }
  };
  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int a0 = (wv >> 1) * 64, b0 = (wv & 1) * 64;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int kc = 0; kc < nch; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nch) load_step(kc + 1);
#pragma unroll
    for (int k16 = 0; k16 < BK; k16 += 16) {
      const b8_t fa0 = lds_frag_b(As[buf], a0 + r32, k16 + kh);
      const b8_t fa1 = lds_frag_b(As[buf], a0 + 32 + r32, k16 + kh);
      const b8_t fb0 = lds_frag_b(Bs[buf], b0 + r32, k16 + kh);
      const b8_t fb1 = lds_frag_b(Bs[buf], b0 + 32 + r32, k16 + kh);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb1, acc[1][1], 0, 0, 0);
    }
    if (kc + 1 < nch) store_step(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + a0 + 32 * mi + acc_row(r, lane);
        const int col = n0 + b0 + 32 * ni + r32;
        if (row < T && col < E) logits[(size_t)row * E + col] = acc[mi][ni][r] + (bias ? bias[col] : 0.0f);
      }
}

hipError_t launch_router_mfma(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s) {
  dim3 grid((T + BM - 1) / BM, (E + BN - 1) / BN);
  hipLaunchKernelGGL(k_router_mfma, grid, dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: split the groups of a permutation between the MFMA GEMM (groups with at
// least min_rows entries, cut into BM-row tiles) and the GEMV work items (the
// rest, items_per entries each).  One block of 1024 threads, thread = group.
// ---------------------------------------------------------------------------
__device__ int plan_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    const int s = wsum[i];
    if (i < w) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ offsets, int E, int min_rows,
                                               int items_per, int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ n_tiles, int32_t* __restrict__ items,
                                               int32_t* __restrict__ n_items) {
  const int G = E + 1;
  const int g = threadIdx.x;
  const int start = g < G ? offsets[g] : 0;
  const int cnt = g < G ? offsets[g + 1] - start : 0;
  const bool big = cnt >= min_rows;
  const int nt = big ? (cnt + BM - 1) / BM : 0;
  const int ni = big ? 0 : (cnt + items_per - 1) / items_per;
  int tot_t = 0, tot_i = 0;
  const int pt = plan_scan_1024(nt, &tot_t);
  const int pi = plan_scan_1024(ni, &tot_i);
  for (int i = 0; i < nt; ++i) {
    tiles[3 * (pt + i)] = g;
    tiles[3 * (pt + i) + 1] = start + i * BM;
    tiles[3 * (pt + i) + 2] = min(BM, cnt - i * BM);
  }
  for (int i = 0; i < ni; ++i) {
    items[3 * (pi + i)] = g;
    items[3 * (pi + i) + 1] = start + i * items_per;
    items[3 * (pi + i) + 2] = min(items_per, cnt - i * items_per);
  }
  if (g == 0) {
    *n_tiles = tot_t;
    *n_items = tot_i;
  }
}

hipError_t launch_plan(const int32_t* offsets, int E, int min_rows, int items_per, int32_t* tiles,
                       int32_t* n_tiles, int32_t* items, int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, s, offsets, E, min_rows, items_per, tiles, n_tiles, items,
                     n_items);
  return hipGetLastError();
}

int gemm_tile_rows() { return BM; }

}  // namespace moe

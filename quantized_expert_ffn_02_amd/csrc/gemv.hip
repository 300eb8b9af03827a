// Dequant-GEMV expert FFN for groups with few tokens (decode, MTP verify).
//
// The pages' decode speed rests on streaming only the selected experts' 2-bit
// weights per token (page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming
// GPU", section "How a 125B model fits in 12 GB"; the Q2_0 build of section
// "The numbers, measured by the author").  Here that stream is HBM-bound: each
// lane owns one weight row, every wave instruction loads 1 KB of codes
// (64 rows x 16 bytes) contiguously, the activations are read as wave-uniform
// scalar loads, and the 2-bit codes become bf16 operands of v_dot2c_f32_bf16
// with one v_and_or_b32 per pair of weights (device.h, "magic pair" form).
// The fp16 block scale is applied once per 32 weights in fp32.
//
// Kernels:
//   k_prep_table_*   activation rows -> per-block pair tables + init values
//   k_gemv_quant     Q2/Q3 GEMV over the groups of a permutation; GateUp mode
//                    computes gate and up rows of a 64-row group and writes
//                    h = SiLU(gate) * up, Down mode writes y rows
//   k_gemv_dense     the same for unquantised bf16 banks (fp32 FMA)
#include <math.h>

#include "device.h"
#include "internal.h"
#include "table.h"

namespace moe {

template <bool Q3>
__global__ __launch_bounds__(256) void k_prep_table_bf16(const uint16_t* __restrict__ x, int K,
                                                         uint32_t* __restrict__ pairs, float* __restrict__ init) {
  const int row = blockIdx.x, nblk = K / 32;
  for (int idx = threadIdx.x; idx < nblk * 16; idx += 256) {
    const int b = idx >> 4, wi = (idx >> 3) & 1, j = idx & 7;
    const int k0 = b * 32 + wi * 16 + j;
    const float v0 = bf16_to_f32(x[(size_t)row * K + k0]);
    const float v1 = bf16_to_f32(x[(size_t)row * K + k0 + 8]);
    prep_row<Q3, false>(v0, v1, row, b, wi, j, nblk, pairs, init);
  }
}

template <bool Q3>
__global__ __launch_bounds__(256) void k_prep_table_f32(const float* __restrict__ h, int K,
                                                        uint32_t* __restrict__ pairs, float* __restrict__ init) {
  const int row = blockIdx.x, nblk = K / 32;
  for (int idx = threadIdx.x; idx < nblk * 16; idx += 256) {
    const int b = idx >> 4, wi = (idx >> 3) & 1, j = idx & 7;
    const int k0 = b * 32 + wi * 16 + j;
    prep_row<Q3, true>(h[(size_t)row * K + k0], h[(size_t)row * K + k0 + 8], row, b, wi, j, nblk, pairs, init);
  }
}

hipError_t launch_prep_table_bf16(const uint16_t* x, int rows, int K, bool q3, uint32_t* pairs, float* init,
                                  hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (q3)
    MOE_LAUNCH(k_prep_table_bf16<true>, dim3(rows), dim3(256), 0, s, x, K, pairs, init);
  else
    MOE_LAUNCH(k_prep_table_bf16<false>, dim3(rows), dim3(256), 0, s, x, K, pairs, init);
  return hipGetLastError();
}

hipError_t launch_prep_table_f32(const float* h, int rows, int K, bool q3, uint32_t* pairs, float* init,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (q3)
    MOE_LAUNCH(k_prep_table_f32<true>, dim3(rows), dim3(256), 0, s, h, K, pairs, init);
  else
    MOE_LAUNCH(k_prep_table_f32<false>, dim3(rows), dim3(256), 0, s, h, K, pairs, init);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_bf16_rows_to_f32(const uint16_t* __restrict__ x, size_t n,
                                                          float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    out[i] = bf16_to_f32(x[i]);
}

hipError_t launch_bf16_rows_to_f32(const uint16_t* x, int rows, int K, float* out, hipStream_t s) {
  const size_t n = (size_t)rows * K;
  if (!n) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  MOE_LAUNCH(k_bf16_rows_to_f32, dim3(blocks), dim3(256), 0, s, x, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Work-item lookup for the dense kernel (the quantized kernel reads the same
// fields from its own __restrict__ arguments).
// ---------------------------------------------------------------------------
struct ItemView {
  int g, start, cnt;
};

__device__ __forceinline__ bool load_item(const PermRef& P, int slot, ItemView& v) {
  if (slot >= __builtin_amdgcn_readfirstlane(*P.n_items)) return false;
  v.g = __builtin_amdgcn_readfirstlane(P.items[3 * slot]);
  v.start = __builtin_amdgcn_readfirstlane(P.items[3 * slot + 1]);
  v.cnt = __builtin_amdgcn_readfirstlane(P.items[3 * slot + 2]);
  return true;
}

// token of sorted position p
__device__ __forceinline__ int token_of(const PermRef& P, int p) {
  const int r = __builtin_amdgcn_readfirstlane(P.sorted_rows[p]);
  const int Tk = P.T * P.k;
  return r < Tk ? r / P.k : r - Tk;
}

// ---------------------------------------------------------------------------
// Quantized GEMV.  grid = (max_groups, row groups), block = W waves; wave w owns
// CPW consecutive 64-column chunks and issues ALL of their code / scale loads
// before any arithmetic, so a block keeps W * CPW KB of codes per matrix in
// flight (HBM latency is paid once, not once per chunk).  The weights stay in
// registers while the group's tokens are processed TB at a time; partial sums
// meet in LDS in wave order.
// ---------------------------------------------------------------------------
// Every pointer is a separate __restrict__ kernel argument: that is what lets
// the compiler prove the activation table is never written by this kernel and
// read it with scalar loads (s_load) instead of per-lane vector loads.
template <GemvKind KIND, bool Q3, int W, int CPW, int TB>
__global__ __launch_bounds__(W * 64) void k_gemv_quant(
    const uint8_t* __restrict__ r_codes, const uint8_t* __restrict__ r_hi, const uint16_t* __restrict__ r_scales,
    const uint8_t* __restrict__ s_codes, const uint8_t* __restrict__ s_hi, const uint16_t* __restrict__ s_scales,
    size_t code_stride, size_t hi_stride, size_t scale_stride, int N, int K, int inter,
    const int32_t* __restrict__ sorted_rows, const int32_t* __restrict__ items,
    const int32_t* __restrict__ n_items, int T, int k, int E,
    const uint32_t* __restrict__ tpairs, const float* __restrict__ tinit, float* __restrict__ out,
    uint32_t* __restrict__ down_pairs, float* __restrict__ down_init, const int32_t* __restrict__ slot_map) {
  constexpr int NMAT = KIND == GemvKind::GateUp ? 2 : 1;
  constexpr bool SPLIT = KIND == GemvKind::Down;
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * (SPLIT ? 2 : 1);
  __shared__ float red[W][NMAT][TB][64];

  const int item = blockIdx.x;
  if (item >= n_items[0]) return;
  const int grp = items[3 * item];
  const int gstart = items[3 * item + 1];
  const int gcnt = items[3 * item + 2];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, provably
  const bool is_shared = grp == E;
  // expert-cache mode: routed expert grp lives in slot slot_map[grp] of the bank, or is a miss
  const int slot = (slot_map && !is_shared) ? slot_map[grp] : grp;
  if (slot < 0) {
    if (KIND == GemvKind::Down) {   // a miss contributes zero to the combine
      for (int i = 0; i < gcnt; ++i)
        for (int c = threadIdx.x; c < 64; c += blockDim.x) out[(size_t)(gstart + i) * N + blockIdx.y * 64 + c] = 0.0f;
    }
    return;
  }
  const size_t eidx = is_shared ? 0 : (size_t)slot;
  const uint4* __restrict__ codes =
      reinterpret_cast<const uint4*>((is_shared ? s_codes : r_codes) + eidx * code_stride);
  const uint32_t* __restrict__ scales =
      reinterpret_cast<const uint32_t*>((is_shared ? s_scales : r_scales) + eidx * scale_stride);
  const uint2* __restrict__ hib =
      Q3 ? reinterpret_cast<const uint2*>((is_shared ? s_hi : r_hi) + eidx * hi_stride) : nullptr;

  const int nch = K / 64, nblk = K / 32, n128 = K / 128;
  int ng[NMAT];
  ng[0] = blockIdx.y;
  if (NMAT == 2) ng[NMAT - 1] = blockIdx.y + inter / 64;
  const int c0 = wv * CPW;

  // ---- all weight loads of this wave first
  uint4 w[NMAT][CPW];
  uint32_t sc[NMAT][CPW];
  uint2 hw[NMAT][CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = c0 + u < nch ? c0 + u : nch - 1;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const size_t tile = (size_t)ng[m] * nch + c;
      w[m][u] = codes[tile * 64 + lane];
      sc[m][u] = scales[(((size_t)ng[m] * n128 + (c >> 1)) * 64 + lane) * 2 + (c & 1)];
      if (Q3) hw[m][u] = hib[tile * 64 + lane];
    }
  }
  const Q2Masks MQ = q2_masks();
  Q3Masks MH;
  if (Q3) MH = q3_masks();

  const int Tk = T * k;
  for (int b0 = 0; b0 < gcnt; b0 += TB) {
    const int nb = min(TB, gcnt - b0);
#pragma unroll 1
    for (int i = 0; i < nb; ++i) {
      const int p = gstart + b0 + i;
      int row = p;
      if (KIND == GemvKind::GateUp) {
        const int r = sorted_rows[p];
        row = r < Tk ? r / k : r - Tk;
      }
      const uint32_t* __restrict__ xrow = tpairs + (size_t)row * nblk * (SETS * 16);
      const float* __restrict__ irow = tinit + (size_t)row * nblk;
      // Keep the code unpacking inside this loop: without this the compiler hoists
      // the unpacked pairs of every chunk out of the token loop and spills them.
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
          asm volatile("" : "+v"(w[m][u].x), "+v"(w[m][u].y), "+v"(w[m][u].z), "+v"(w[m][u].w));
          if (Q3) asm volatile("" : "+v"(hw[m][u].x), "+v"(hw[m][u].y));
        }
      float acc[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const uint32_t* __restrict__ xp = xrow + (size_t)(2 * c) * (SETS * 16);
          const float i0 = irow[2 * c], i1 = irow[2 * c + 1];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            float a0 = i0, a1 = i1;
#pragma unroll
            for (int s = 0; s < (SPLIT ? 2 : 1); ++s) {
              const uint32_t* __restrict__ x0 = xp + (s * PLANES) * 16;
              const uint32_t* __restrict__ x1 = xp + SETS * 16 + (s * PLANES) * 16;
              a0 = q2_word_dot(w[m][u].x, x0, a0, MQ);
              a0 = q2_word_dot(w[m][u].y, x0 + 8, a0, MQ);
              a1 = q2_word_dot(w[m][u].z, x1, a1, MQ);
              a1 = q2_word_dot(w[m][u].w, x1 + 8, a1, MQ);
              if (Q3) {
                a0 = q3_hi_dot(hw[m][u].x, x0 + 16, a0, MH);
                a0 = q3_hi_dot(hw[m][u].x >> 8, x0 + 24, a0, MH);
                a1 = q3_hi_dot(hw[m][u].y, x1 + 16, a1, MH);
                a1 = q3_hi_dot(hw[m][u].y >> 8, x1 + 24, a1, MH);
              }
            }
            acc[m] = fmaf(fp16_to_f32(sc[m][u] & 0xFFFFu), a0, acc[m]);
            acc[m] = fmaf(fp16_to_f32(sc[m][u] >> 16), a1, acc[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) red[wv][m][i][lane] = acc[m];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (i < nb) {
          float v[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            float s = red[0][m][i][lane];
            for (int u = 1; u < W; ++u) s += red[u][m][i][lane];
            v[m] = s;
          }
          const size_t p = (size_t)(gstart + b0 + i);
          if (KIND == GemvKind::GateUp) {
            const float a = v[0], b = v[NMAT - 1];
            const float hv = a / (1.0f + expf(-a)) * b;
            if (down_pairs)
              emit_down_table<Q3>(hv, (int)p, blockIdx.y, inter, down_pairs, down_init);
            else
              out[p * inter + (size_t)blockIdx.y * 64 + lane] = hv;
          } else {
            out[p * N + (size_t)blockIdx.y * 64 + lane] = v[0];
          }
        }
      }
    }
    __syncthreads();
  }
}

// Launch shapes with their own register budgets: gate/up 8 waves x 5 chunks
// (K = 2560), down 5 waves x 2 chunks (K = 640); other K use 8 waves of up to
// 5 chunks, and 16 waves x 4 chunks beyond K = 2560.
template <GemvKind KIND, bool Q3>
static hipError_t launch_quant_t(const MatRef& r, const MatRef& sh, int N, int K, int inter, const PermRef& P,
                                 int max_groups, const TableRef& tab, float* out, uint32_t* dp, float* di,
                                 hipStream_t s) {
  const int rowgroups = KIND == GemvKind::GateUp ? inter / 64 : N / 64;
  const int nch = K / 64;
  dim3 grid(max_groups, rowgroups);
#define MOE_GEMV_ARGS                                                                                          \
  r.codes, r.hi, r.scales, sh.codes, sh.hi, sh.scales, r.code_stride, r.hi_stride, r.scale_stride, N, K, inter, \
      P.sorted_rows, P.items, P.n_items, P.T, P.k, P.E, tab.pairs, tab.init, out, dp, di, P.slot_map
  if (KIND == GemvKind::GateUp && nch == 40) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 8, 5, 4>), grid, dim3(512), 0, s, MOE_GEMV_ARGS);
  } else if (KIND == GemvKind::Down && nch == 10) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 5, 2, 4>), grid, dim3(320), 0, s, MOE_GEMV_ARGS);
  } else if (nch <= 8) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 8, 1, 4>), grid, dim3(512), 0, s, MOE_GEMV_ARGS);
  } else if (nch <= 16) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 8, 2, 4>), grid, dim3(512), 0, s, MOE_GEMV_ARGS);
  } else if (nch <= 40) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 8, 5, 4>), grid, dim3(512), 0, s, MOE_GEMV_ARGS);
  } else if (nch <= 64) {
    MOE_LAUNCH((k_gemv_quant<KIND, Q3, 16, 4, 4>), grid, dim3(1024), 0, s, MOE_GEMV_ARGS);
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_GEMV_ARGS
  return hipGetLastError();
}

hipError_t launch_gemv_quant(GemvKind kind, int fmt, const MatRef& routed, const MatRef& shared, int N, int K,
                             int inter, const PermRef& perm, int max_groups, const TableRef& tab, float* out,
                             uint32_t* down_pairs, float* down_init, hipStream_t s) {
  if (max_groups <= 0) return hipSuccess;
  const bool q3 = fmt == MOE_FMT_Q3;
  if (kind == GemvKind::GateUp)
    return q3 ? launch_quant_t<GemvKind::GateUp, true>(routed, shared, N, K, inter, perm, max_groups, tab, out,
                                                       down_pairs, down_init, s)
              : launch_quant_t<GemvKind::GateUp, false>(routed, shared, N, K, inter, perm, max_groups, tab, out,
                                                        down_pairs, down_init, s);
  return q3 ? launch_quant_t<GemvKind::Down, true>(routed, shared, N, K, inter, perm, max_groups, tab, out,
                                                   nullptr, nullptr, s)
            : launch_quant_t<GemvKind::Down, false>(routed, shared, N, K, inter, perm, max_groups, tab, out,
                                                    nullptr, nullptr, s);
}

// ---------------------------------------------------------------------------
// Unquantised (bf16) banks: same grid, lane = row, 8 bf16 per 16-byte chunk,
// fp32 FMA against fp32 input rows read as wave-uniform values.
// ---------------------------------------------------------------------------
template <GemvKind KIND, int W>
__global__ __launch_bounds__(W * 64) void k_gemv_dense(MatRef routed, MatRef shared, int N, int K, int inter,
                                                       PermRef P, const float* __restrict__ in_rows,
                                                       float* __restrict__ out) {
  constexpr int NMAT = KIND == GemvKind::GateUp ? 2 : 1;
  __shared__ float red[W][NMAT][64];
  ItemView G;
  if (!load_item(P, blockIdx.x, G)) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool is_shared = G.g == P.E;
  const MatRef& M = is_shared ? shared : routed;
  const size_t eidx = is_shared ? 0 : (size_t)G.g;
  const uint4* __restrict__ wv16 = reinterpret_cast<const uint4*>(M.codes + eidx * M.code_stride);
  const int nch = K / 8;
  int ng[NMAT];
  ng[0] = blockIdx.y;
  if (NMAT == 2) ng[NMAT - 1] = blockIdx.y + inter / 64;
  const int cpw = (nch + W - 1) / W;
  const int c0 = wv * cpw, c1 = min(nch, c0 + cpw);
  for (int e = 0; e < G.cnt; ++e) {
    const int p = G.start + e;
    const int row = KIND == GemvKind::GateUp ? token_of(P, p) : p;
    const float* __restrict__ xr = in_rows + (size_t)row * K;
    float acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = 0.0f;
    for (int c = c0; c < c1; ++c) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint4 q = wv16[((size_t)ng[m] * nch + c) * 64 + lane];
        const uint32_t ww[4] = {q.x, q.y, q.z, q.w};
        float a = acc[m];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a = fmaf(bf16_to_f32(ww[u] & 0xFFFFu), xr[c * 8 + 2 * u], a);
          a = fmaf(bf16_to_f32(ww[u] >> 16), xr[c * 8 + 2 * u + 1], a);
        }
        acc[m] = a;
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m) red[wv][m][lane] = acc[m];
    __syncthreads();
    if (wv == 0) {
      float v[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float s = red[0][m][lane];
        for (int u = 1; u < W; ++u) s += red[u][m][lane];
        v[m] = s;
      }
      if (KIND == GemvKind::GateUp) {
        const float a = v[0], b = v[NMAT - 1];
        out[(size_t)p * inter + (size_t)blockIdx.y * 64 + lane] = a / (1.0f + expf(-a)) * b;
      } else {
        out[(size_t)p * N + (size_t)blockIdx.y * 64 + lane] = v[0];
      }
    }
    __syncthreads();
  }
}

hipError_t launch_gemv_dense(GemvKind kind, const MatRef& routed, const MatRef& shared, int N, int K, int inter,
                             const PermRef& perm, int max_groups, const float* in_rows, float* out,
                             hipStream_t s) {
  if (max_groups <= 0) return hipSuccess;
  if (kind == GemvKind::GateUp)
    MOE_LAUNCH((k_gemv_dense<GemvKind::GateUp, 4>), dim3(max_groups, inter / 64), dim3(256), 0, s, routed,
                       shared, N, K, inter, perm, in_rows, out);
  else
    MOE_LAUNCH((k_gemv_dense<GemvKind::Down, 2>), dim3(max_groups, N / 64), dim3(128), 0, s, routed,
                       shared, N, K, inter, perm, in_rows, out);
  return hipGetLastError();
}

}  // namespace moe

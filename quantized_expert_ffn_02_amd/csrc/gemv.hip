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

namespace moe {

// exponent shift p of lo-plane pair j and q of hi-plane pair j (device.h tables)
__device__ __forceinline__ int lo_shift(int j) {
  const int P[8] = {0, 2, 4, 0, 2, 4, 0, 2};
  return P[j];
}
__device__ __forceinline__ int hi_shift(int j) { return j < 7 ? j : 0; }

// ---------------------------------------------------------------------------
// Activation tables.  One block of 256 threads per input row; 16 threads per
// 32-column block: thread (wi, j) handles the pair (16 wi + j, 16 wi + j + 8).
// Sets per block: [split][plane] with split = hi, lo (fp32 input only) and
// plane = lo codes, hi bits (Q3 only).
// ---------------------------------------------------------------------------
template <bool Q3, bool SPLIT>
__device__ void prep_row(const float v0, const float v1, int row, int b, int wi, int j, int nblk,
                         uint32_t* __restrict__ pairs, float* __restrict__ init) {
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * (SPLIT ? 2 : 1);
  const float sp = ldexpf(1.0f, -lo_shift(j));
  const float sq = ldexpf(4.0f, -hi_shift(j));
  float hi0 = v0, hi1 = v1, lo0 = 0.0f, lo1 = 0.0f;
  if (SPLIT) {
    hi0 = bf16_to_f32(f32_to_bf16_rne(v0));
    hi1 = bf16_to_f32(f32_to_bf16_rne(v1));
    lo0 = bf16_to_f32(f32_to_bf16_rne(v0 - hi0));
    lo1 = bf16_to_f32(f32_to_bf16_rne(v1 - hi1));
  }
  uint32_t* __restrict__ dst = pairs + ((size_t)row * nblk + b) * (SETS * 16) + wi * 8 + j;
  const float parts0[2] = {hi0, lo0}, parts1[2] = {hi1, lo1};
#pragma unroll
  for (int s = 0; s < (SPLIT ? 2 : 1); ++s) {
    dst[(s * PLANES) * 16] = f32_to_bf16_rne(parts0[s] * sp) | (f32_to_bf16_rne(parts1[s] * sp) << 16);
    if (Q3)
      dst[(s * PLANES + 1) * 16] = f32_to_bf16_rne(parts0[s] * sq) | (f32_to_bf16_rne(parts1[s] * sq) << 16);
  }
  // init = -sum_k (128 2^-p + [512 2^-q] + offset) * value_k over the block's 32 weights
  const float mult = 128.0f * sp + (Q3 ? 128.0f * sq + 4.0f : 2.0f);
  float term = mult * (hi0 + lo0) + mult * (hi1 + lo1);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) term += __shfl_xor(term, off, 16);
  if (wi == 0 && j == 0) init[(size_t)row * nblk + b] = -term;
}

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
    hipLaunchKernelGGL(k_prep_table_bf16<true>, dim3(rows), dim3(256), 0, s, x, K, pairs, init);
  else
    hipLaunchKernelGGL(k_prep_table_bf16<false>, dim3(rows), dim3(256), 0, s, x, K, pairs, init);
  return hipGetLastError();
}

hipError_t launch_prep_table_f32(const float* h, int rows, int K, bool q3, uint32_t* pairs, float* init,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (q3)
    hipLaunchKernelGGL(k_prep_table_f32<true>, dim3(rows), dim3(256), 0, s, h, K, pairs, init);
  else
    hipLaunchKernelGGL(k_prep_table_f32<false>, dim3(rows), dim3(256), 0, s, h, K, pairs, init);
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
  hipLaunchKernelGGL(k_bf16_rows_to_f32, dim3(blocks), dim3(256), 0, s, x, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Group lookup shared by the GEMV kernels.
// ---------------------------------------------------------------------------
struct GroupView {
  int g, start, cnt;
};

__device__ __forceinline__ bool load_group(const PermRef& P, int slot, GroupView& v) {
  if (slot >= __builtin_amdgcn_readfirstlane(*P.n_active)) return false;
  v.g = __builtin_amdgcn_readfirstlane(P.active[slot]);
  v.start = __builtin_amdgcn_readfirstlane(P.offsets[v.g]);
  v.cnt = __builtin_amdgcn_readfirstlane(P.offsets[v.g + 1]) - v.start;
  return true;
}

// token of sorted position p
__device__ __forceinline__ int token_of(const PermRef& P, int p) {
  const int r = __builtin_amdgcn_readfirstlane(P.sorted_rows[p]);
  const int Tk = P.T * P.k;
  return r < Tk ? r / P.k : r - Tk;
}

// ---------------------------------------------------------------------------
// Quantized GEMV.  grid = (max_groups, row groups), block = W waves; wave w
// covers a contiguous range of the 64-column chunks; tokens of the group are
// processed TB at a time; partial sums meet in LDS in wave order.
// ---------------------------------------------------------------------------
template <GemvKind KIND, bool Q3, int W, int TB>
__global__ __launch_bounds__(W * 64) void k_gemv_quant(MatRef routed, MatRef shared, int N, int K, int inter,
                                                       PermRef P, TableRef tab, float* __restrict__ out) {
  constexpr int NMAT = KIND == GemvKind::GateUp ? 2 : 1;
  constexpr bool SPLIT = KIND == GemvKind::Down;
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * (SPLIT ? 2 : 1);
  __shared__ float red[W][NMAT][TB][64];

  GroupView G;
  if (!load_group(P, blockIdx.x, G)) return;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const bool is_shared = G.g == P.E;
  const MatRef& M = is_shared ? shared : routed;
  const size_t eidx = is_shared ? 0 : (size_t)G.g;
  const uint4* __restrict__ codes = reinterpret_cast<const uint4*>(M.codes + eidx * M.code_stride);
  const uint32_t* __restrict__ scales = reinterpret_cast<const uint32_t*>(M.scales + eidx * M.scale_stride);
  const uint2* __restrict__ hib = Q3 ? reinterpret_cast<const uint2*>(M.hi + eidx * M.hi_stride) : nullptr;

  const int nch = K / 64, nblk = K / 32, n128 = K / 128;
  int ng[NMAT];
  ng[0] = blockIdx.y;
  if (NMAT == 2) ng[NMAT - 1] = blockIdx.y + inter / 64;
  const int cpw = (nch + W - 1) / W;
  const int c0 = wv * cpw, c1 = min(nch, c0 + cpw);
  const Q2Masks MQ = q2_masks();
  Q3Masks MH;
  if (Q3) MH = q3_masks();

  for (int b0 = 0; b0 < G.cnt; b0 += TB) {
    const int nb = min(TB, G.cnt - b0);
    int rows[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int p = G.start + b0 + (i < nb ? i : 0);
      rows[i] = KIND == GemvKind::GateUp ? token_of(P, p) : p;
    }
    float acc[NMAT][TB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < TB; ++i) acc[m][i] = 0.0f;

    for (int c = c0; c < c1; ++c) {
      uint4 w[NMAT];
      uint32_t sc[NMAT];
      uint2 hw[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const size_t tile = (size_t)ng[m] * nch + c;
        w[m] = codes[tile * 64 + lane];
        sc[m] = scales[(((size_t)ng[m] * n128 + (c >> 1)) * 64 + lane) * 2 + (c & 1)];
        if (Q3) hw[m] = hib[tile * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (i < nb) {
          const uint32_t* __restrict__ xp = tab.pairs + ((size_t)rows[i] * nblk + 2 * c) * (SETS * 16);
          const float i0 = tab.init[(size_t)rows[i] * nblk + 2 * c];
          const float i1 = tab.init[(size_t)rows[i] * nblk + 2 * c + 1];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            float a0 = i0, a1 = i1;
#pragma unroll
            for (int s = 0; s < (SPLIT ? 2 : 1); ++s) {
              const uint32_t* __restrict__ x0 = xp + (s * PLANES) * 16;
              const uint32_t* __restrict__ x1 = xp + SETS * 16 + (s * PLANES) * 16;
              a0 = q2_word_dot(w[m].x, x0, a0, MQ);
              a0 = q2_word_dot(w[m].y, x0 + 8, a0, MQ);
              a1 = q2_word_dot(w[m].z, x1, a1, MQ);
              a1 = q2_word_dot(w[m].w, x1 + 8, a1, MQ);
              if (Q3) {
                a0 = q3_hi_dot(hw[m].x, x0 + 16, a0, MH);
                a0 = q3_hi_dot(hw[m].x >> 8, x0 + 24, a0, MH);
                a1 = q3_hi_dot(hw[m].y, x1 + 16, a1, MH);
                a1 = q3_hi_dot(hw[m].y >> 8, x1 + 24, a1, MH);
              }
            }
            acc[m][i] = fmaf(fp16_to_f32(sc[m] & 0xFFFFu), a0, acc[m][i]);
            acc[m][i] = fmaf(fp16_to_f32(sc[m] >> 16), a1, acc[m][i]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < TB; ++i) red[wv][m][i][lane] = acc[m][i];
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
          const size_t p = (size_t)(G.start + b0 + i);
          if (KIND == GemvKind::GateUp) {
            const float a = v[0], b = v[NMAT - 1];
            out[p * inter + (size_t)blockIdx.y * 64 + lane] = a / (1.0f + expf(-a)) * b;
          } else {
            out[p * N + (size_t)blockIdx.y * 64 + lane] = v[0];
          }
        }
      }
    }
    __syncthreads();
  }
}

template <GemvKind KIND, bool Q3, int W>
static void launch_quant_t(const MatRef& r, const MatRef& sh, int N, int K, int inter, const PermRef& P,
                           int max_groups, const TableRef& tab, float* out, hipStream_t s) {
  const int rowgroups = KIND == GemvKind::GateUp ? inter / 64 : N / 64;
  hipLaunchKernelGGL((k_gemv_quant<KIND, Q3, W, 4>), dim3(max_groups, rowgroups), dim3(W * 64), 0, s, r, sh, N, K,
                     inter, P, tab, out);
}

hipError_t launch_gemv_quant(GemvKind kind, int fmt, const MatRef& routed, const MatRef& shared, int N, int K,
                             int inter, const PermRef& perm, int max_groups, const TableRef& tab, float* out,
                             hipStream_t s) {
  if (max_groups <= 0) return hipSuccess;
  const bool q3 = fmt == MOE_FMT_Q3;
  if (kind == GemvKind::GateUp) {
    if (q3)
      launch_quant_t<GemvKind::GateUp, true, 4>(routed, shared, N, K, inter, perm, max_groups, tab, out, s);
    else
      launch_quant_t<GemvKind::GateUp, false, 4>(routed, shared, N, K, inter, perm, max_groups, tab, out, s);
  } else {
    if (q3)
      launch_quant_t<GemvKind::Down, true, 2>(routed, shared, N, K, inter, perm, max_groups, tab, out, s);
    else
      launch_quant_t<GemvKind::Down, false, 2>(routed, shared, N, K, inter, perm, max_groups, tab, out, s);
  }
  return hipGetLastError();
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
  GroupView G;
  if (!load_group(P, blockIdx.x, G)) return;
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
    hipLaunchKernelGGL((k_gemv_dense<GemvKind::GateUp, 4>), dim3(max_groups, inter / 64), dim3(256), 0, s, routed,
                       shared, N, K, inter, perm, in_rows, out);
  else
    hipLaunchKernelGGL((k_gemv_dense<GemvKind::Down, 2>), dim3(max_groups, N / 64), dim3(128), 0, s, routed,
                       shared, N, K, inter, perm, in_rows, out);
  return hipGetLastError();
}

}  // namespace moe

// Gate-weighted combine of the expert outputs plus the shared expert, in a
// fixed order (no atomics), with an optional residual add and bf16 copy.
// The shared expert is added with weight 1 for every token (page "Strata Runs
// 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "What it is": one
// shared expert fires per token).  A fixed summation order makes the output
// the same on every run, the property the pages report for the engine's
// releases (page "Strata: a 125B AI model on your gaming PC", section "What is
// new in Strata 0.1.45": byte-identical answers).
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace moe {

// Loads are issued a batch of kCombineBatch entries at a time (indices clamped
// to the last entry, extra values dropped) and then added in entry order, so a
// thread waits for one memory round trip per batch instead of one per entry.
static constexpr int kCombineBatch = 12;

// Outputs 4q .. 4q + 3 of token row t: sum_i g_i y_i in rank order, the shared
// expert's row, then the residual (bf16), in fp32.
__device__ __forceinline__ float4 combine4(const float* __restrict__ y_sorted, const int32_t* __restrict__ row_to_sorted,
                                           const float* __restrict__ gates, int T, int k, int H, int with_shared,
                                           const uint16_t* __restrict__ residual, int t, int q) {
  const size_t H4 = H / 4;
  uint2 rb = make_uint2(0u, 0u);
  if (residual) rb = reinterpret_cast<const uint2*>(residual + (size_t)t * H)[q];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int n = k + (with_shared ? 1 : 0);
  for (int i0 = 0; i0 < n; i0 += kCombineBatch) {
    float4 y[kCombineBatch];
    float g[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const int i = i0 + j < n ? i0 + j : n - 1;
      const size_t r = i < k ? (size_t)t * k + i : (size_t)T * k + t;
      g[j] = i < k ? gates[r] : 1.0f;
      y[j] = reinterpret_cast<const float4*>(y_sorted)[(size_t)row_to_sorted[r] * H4 + q];
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (i0 + j < k) {
        acc.x = fmaf(g[j], y[j].x, acc.x);
        acc.y = fmaf(g[j], y[j].y, acc.y);
        acc.z = fmaf(g[j], y[j].z, acc.z);
        acc.w = fmaf(g[j], y[j].w, acc.w);
      } else if (i0 + j < n) {   // the shared expert, weight 1
        acc.x += y[j].x;
        acc.y += y[j].y;
        acc.z += y[j].z;
        acc.w += y[j].w;
      }
    }
  }
  if (residual) {
    acc.x += bf16_to_f32(rb.x & 0xFFFFu);
    acc.y += bf16_to_f32(rb.x >> 16);
    acc.z += bf16_to_f32(rb.y & 0xFFFFu);
    acc.w += bf16_to_f32(rb.y >> 16);
  }
  return acc;
}

__global__ __launch_bounds__(1024) void k_combine(const float* __restrict__ y_sorted,
                                                 const int32_t* __restrict__ row_to_sorted,
                                                 const float* __restrict__ gates, int T, int k, int H,
                                                 int with_shared, const uint16_t* __restrict__ residual,
                                                 float* __restrict__ out, uint16_t* __restrict__ out_bf16) {
  const int t = blockIdx.y;
  const int q = blockIdx.x * blockDim.x + threadIdx.x;   // index of 4 consecutive outputs
  if (q * 4 >= H) return;
  const float4 acc = combine4(y_sorted, row_to_sorted, gates, T, k, H, with_shared, residual, t, q);
  reinterpret_cast<float4*>(out)[(size_t)t * (H / 4) + q] = acc;
  if (out_bf16) {
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(out_bf16 + (size_t)t * H)[q] = o;
  }
}

hipError_t launch_combine(const float* y_sorted, const int32_t* row_to_sorted, const float* gates, int T, int k,
                          int H, int with_shared, const uint16_t* residual, float* out, uint16_t* out_bf16,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // one block per token row when it fits (no partly idle second block)
  const int threads = ((H / 4 + 63) / 64) * 64;
  const dim3 block(threads <= 1024 ? threads : 256);
  dim3 grid((H / 4 + block.x - 1) / block.x, T);
  MOE_LAUNCH(k_combine, grid, block, 0, s, y_sorted, row_to_sorted, gates, T, k, H, with_shared, residual, out,
             out_bf16);
  return hipGetLastError();
}

// The same combine over fp16 rows that already carry their gate (the prompt
// path's down GEMM writes them in the scale of their token's row, y 4^a):
// out[t] = 4^-a (sum_i y16[row_to_sorted[t k + i]] (i = 0..k-1) +
// y16[row_to_sorted[T k + t]]) (+ residual), summed in fp32 in that order.
// Eight consecutive outputs per thread.
__global__ __launch_bounds__(1024) void k_combine16(const uint16_t* __restrict__ y16,
                                                   const int32_t* __restrict__ row_to_sorted, int T, int k, int H,
                                                   int with_shared, const uint16_t* __restrict__ residual,
                                                   float* __restrict__ out, uint16_t* __restrict__ out_bf16,
                                                   const int32_t* __restrict__ xexp) {
  const int t = blockIdx.y;
  const int q = blockIdx.x * blockDim.x + threadIdx.x;   // index of 8 consecutive outputs
  if (q * 8 >= H) return;
  const int ue = xexp ? -2 * xexp[t] : 0;
  const size_t H8 = H / 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  uint4 rb = make_uint4(0u, 0u, 0u, 0u);
  if (residual) rb = reinterpret_cast<const uint4*>(residual + (size_t)t * H)[q];
  const int n = k + (with_shared ? 1 : 0);
  for (int i0 = 0; i0 < n; i0 += kCombineBatch) {
    uint4 v[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const int i = i0 + j < n ? i0 + j : n - 1;
      const size_t r = i < k ? (size_t)t * k + i : (size_t)T * k + t;
      v[j] = reinterpret_cast<const uint4*>(y16)[(size_t)row_to_sorted[r] * H8 + q];
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (i0 + j < n) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] += fp16_to_f32(w[h] & 0xFFFFu);
          acc[2 * h + 1] += fp16_to_f32(w[h] >> 16);
        }
      }
    }
  }
  // the rows were computed for x 2^a: the sum is y 4^a
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = ldexpf(acc[j], ue);
  if (residual) {
    const uint32_t w[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(w[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(w[j] >> 16);
    }
  }
  float4* o = reinterpret_cast<float4*>(out + (size_t)t * H) + 2 * q;
  o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (out_bf16) {
    uint4 b;
    b.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    b.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    b.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    b.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    reinterpret_cast<uint4*>(out_bf16 + (size_t)t * H)[q] = b;
  }
}

hipError_t launch_combine16(const uint16_t* y16, const int32_t* row_to_sorted, int T, int k, int H, int with_shared,
                            const uint16_t* residual, float* out, uint16_t* out_bf16, const int32_t* xexp,
                            hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // one block per token row when it fits (no partly idle second block)
  const int threads = ((H / 8 + 63) / 64) * 64;
  const dim3 block(threads <= 1024 ? threads : 256);
  dim3 grid((H / 8 + block.x - 1) / block.x, T);
  MOE_LAUNCH(k_combine16, grid, block, 0, s, y16, row_to_sorted, T, k, H, with_shared, residual, out, out_bf16,
             xexp);
  return hipGetLastError();
}

// Parameter-free RMSNorm of each bf16 row: bf16(x / sqrt(mean(x^2) + eps)), one
// block per row, fixed-order fp32 reduction (the input of every layer of a stack).
// Rows whose width is a multiple of 8 and at most 8,192: one 16-byte chunk per
// thread (blockDim = H / 8 rounded up to whole waves), loaded once and kept in
// registers for the scaling pass.  Other widths: one element per thread and
// step.
__device__ __forceinline__ float block_sum_fixed(float v, float* part, int nw) {
  v = wave_sum(v);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) part[tid >> 6] = v;
  __syncthreads();
  float tot = 0.0f;
  for (int i = 0; i < nw; ++i) tot += part[i];
  return tot;
}

// RMSNorm of one bf16 row (value of column c: get(c)) of H = 64 G columns
// (G <= 64) with the 64-column group sums (rms_group_sum, lane = column, one wave
// per group) and their total (rms_inv_from_groups, lane = group): out_row =
// bf16(x * inv), rounded to nearest even; the definition the fused stack path
// uses too.  With f16p, also the grouped GEMMs' fp16 copy of the output row
// scaled by its row exponent a (bf16_row_exponent of the output's largest
// magnitude; a written to xexp[row]) in pair order (u32 j of each 16-column
// group = columns j and j + 8), the same bits k_x_to_f16_rows makes from the
// bf16 row.  Every thread of the block calls it; part holds G <= 64 floats,
// wmax 16 words.
template <class Get>
__device__ __forceinline__ void rms_norm_row_g64(Get get, int H, float eps, float* part, uint32_t* wmax,
                                                 uint16_t* __restrict__ out_row, uint32_t* __restrict__ f16p,
                                                 int32_t* __restrict__ xexp, size_t row) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int G = H / 64;
  for (int g = w; g < G; g += nw) {
    const float s = rms_group_sum(get(64 * g + lane));
    if (lane == 0) part[g] = s;
  }
  __syncthreads();
  const float inv = rms_inv_from_groups(lane < G ? part[lane] : 0.0f, H, eps);
  uint32_t m = 0;
  for (int g = w; g < G; g += nw) {
    const uint16_t o = __builtin_bit_cast(uint16_t, (__bf16)(get(64 * g + lane) * inv));
    out_row[64 * g + lane] = o;
    m = max(m, (uint32_t)(o & 0x7FFFu));
  }
  if (!f16p) return;
  m = wave_max_u32(m);
  if (lane == 0) wmax[w] = m;
  __syncthreads();
  for (int i = 0; i < nw; ++i) m = max(m, wmax[i]);
  const int a = bf16_row_exponent(m);
  if (threadIdx.x == 0) xexp[row] = a;
  for (int g = w; g < G; g += nw) {
    const __bf16 o = (__bf16)(get(64 * g + lane) * inv);
    // column + 8 of the same 16-column group: rotate the 16-lane row by 8
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)ldexpf((float)o, a));
    const uint32_t h8 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x128, 0xF, 0xF, true);
    if ((lane & 15) < 8) f16p[(row * H + 64 * g + lane) / 16 * 8 + (lane & 7)] = h | (h8 << 16);
  }
}

__global__ __launch_bounds__(1024) void k_rmsnorm_bf16_g64(const uint16_t* __restrict__ x, int H, float eps,
                                                           uint16_t* __restrict__ out, uint32_t* __restrict__ f16p,
                                                           int32_t* __restrict__ xexp) {
  __shared__ float part[64];
  __shared__ uint32_t wmax[16];
  const int row = blockIdx.x;
  const uint16_t* __restrict__ xr = x + (size_t)row * H;
  rms_norm_row_g64([&](int c) { return bf16_to_f32(xr[c]); }, H, eps, part, wmax, out + (size_t)row * H, f16p, xexp,
                   (size_t)row);
}

// The combine of a stack layer followed by the next layer's RMSNorm of its bf16
// result, one block of H / 4 threads per token row (H % 256 == 0, H <= 4096): the
// row goes through LDS to the norm, which runs exactly as k_rmsnorm_bf16_g64.
__global__ __launch_bounds__(1024) void k_combine_norm(const float* __restrict__ y_sorted,
                                                      const int32_t* __restrict__ row_to_sorted,
                                                      const float* __restrict__ gates, int T, int k, int H,
                                                      int with_shared, const uint16_t* __restrict__ residual,
                                                      float* __restrict__ out, uint16_t* __restrict__ out_bf16,
                                                      float eps, uint16_t* __restrict__ xn, uint32_t* __restrict__ f16p,
                                                      int32_t* __restrict__ xexp) {
  __shared__ float xs[4096];
  __shared__ float part[64];
  __shared__ uint32_t wmax[16];
  const int t = blockIdx.x, q = threadIdx.x;
  const float4 acc = combine4(y_sorted, row_to_sorted, gates, T, k, H, with_shared, residual, t, q);
  if (out) reinterpret_cast<float4*>(out)[(size_t)t * (H / 4) + q] = acc;
  const uint32_t b0 = f32_to_bf16_rne(acc.x), b1 = f32_to_bf16_rne(acc.y);
  const uint32_t b2 = f32_to_bf16_rne(acc.z), b3 = f32_to_bf16_rne(acc.w);
  reinterpret_cast<uint2*>(out_bf16 + (size_t)t * H)[q] = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  *reinterpret_cast<float4*>(xs + 4 * q) = make_float4(bf16_to_f32(b0), bf16_to_f32(b1), bf16_to_f32(b2),
                                                       bf16_to_f32(b3));
  __syncthreads();
  rms_norm_row_g64([&](int c) { return xs[c]; }, H, eps, part, wmax, xn + (size_t)t * H, f16p, xexp, (size_t)t);
}

__global__ __launch_bounds__(1024) void k_rmsnorm_bf16_v8(const uint16_t* __restrict__ x, int H, float eps,
                                                          uint16_t* __restrict__ out) {
  __shared__ float part[16];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nc = H / 8;
  const uint4* __restrict__ xr = reinterpret_cast<const uint4*>(x + (size_t)row * H);
  const uint4 v = tid < nc ? xr[tid] : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8], ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
    f[2 * j + 1] = bf16_to_f32(w[j] >> 16);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(f[j], f[j], ss);
  const float tot = block_sum_fixed(ss, part, (int)(blockDim.x >> 6));
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  if (tid < nc) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_rne(f[2 * j] * inv) | (f32_to_bf16_rne(f[2 * j + 1] * inv) << 16);
    reinterpret_cast<uint4*>(out + (size_t)row * H)[tid] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void k_rmsnorm_bf16(const uint16_t* __restrict__ x, int H, float eps,
                                                      uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* __restrict__ xr = x + (size_t)row * H;
  float ss = 0.0f;
  for (int h = tid; h < H; h += 256) {
    const float v = bf16_to_f32(xr[h]);
    ss = fmaf(v, v, ss);
  }
  const float tot = block_sum_fixed(ss, part, 4);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int h = tid; h < H; h += 256) out[(size_t)row * H + h] = f32_to_bf16_rne(bf16_to_f32(xr[h]) * inv);
}

hipError_t launch_rmsnorm_bf16(const uint16_t* x, int T, int H, float eps, uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 64 == 0 && H / 64 <= 64) {
    const int G = H / 64;
    MOE_LAUNCH(k_rmsnorm_bf16_g64, dim3(T), dim3(64 * (G < 16 ? G : 16)), 0, s, x, H, eps, out,
               (uint32_t*)nullptr, (int32_t*)nullptr);
  } else if (H % 8 == 0 && H <= 8192) {
    const int threads = ((H / 8 + 63) / 64) * 64;
    MOE_LAUNCH(k_rmsnorm_bf16_v8, dim3(T), dim3(threads), 0, s, x, H, eps, out);
  } else {
    MOE_LAUNCH(k_rmsnorm_bf16, dim3(T), dim3(256), 0, s, x, H, eps, out);
  }
  return hipGetLastError();
}

bool rmsnorm_f16_pairs_ok(int H) { return H % 64 == 0 && H / 64 <= 64; }

bool combine_norm_ok(int H) { return H % 256 == 0 && H <= 4096; }

hipError_t launch_combine_norm(const float* y_sorted, const int32_t* row_to_sorted, const float* gates, int T, int k,
                               int H, int with_shared, const uint16_t* residual, float* out, uint16_t* out_bf16,
                               float eps, uint16_t* xn, uint16_t* f16p, int32_t* xexp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!combine_norm_ok(H) || !out_bf16 || !xn || (f16p && !xexp)) return hipErrorInvalidValue;
  MOE_LAUNCH(k_combine_norm, dim3(T), dim3(H / 4), 0, s, y_sorted, row_to_sorted, gates, T, k, H, with_shared,
             residual, out, out_bf16, eps, xn, reinterpret_cast<uint32_t*>(f16p), xexp);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16_f16pairs(const uint16_t* x, int T, int H, float eps, uint16_t* out, uint16_t* f16p,
                                        int32_t* xexp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!rmsnorm_f16_pairs_ok(H) || !xexp) return hipErrorInvalidValue;
  const int G = H / 64;
  MOE_LAUNCH(k_rmsnorm_bf16_g64, dim3(T), dim3(64 * (G < 16 ? G : 16)), 0, s, x, H, eps, out,
             reinterpret_cast<uint32_t*>(f16p), xexp);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_workspace_clear(void* ws, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  MOE_LAUNCH(k_fill_zero, dim3(blocks), dim3(256), 0, s, (uint32_t*)ws, n);
  return hipGetLastError();
}

// out[i] += y[i] for i < n (the tiered layer adds the host-computed miss sum to the
// GPU's hits + shared output).  float4 for the bulk, scalars for a tail.
__global__ __launch_bounds__(256) void k_add_f32(float* __restrict__ out, const float* __restrict__ y, size_t n) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 a = reinterpret_cast<float4*>(out)[i];
    const float4 b = reinterpret_cast<const float4*>(y)[i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
    reinterpret_cast<float4*>(out)[i] = a;
  }
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] += y[i];
}

hipError_t launch_add_f32(float* out, const float* y, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (((uintptr_t)out | (uintptr_t)y) & 15) return hipErrorInvalidValue;
  const size_t want = (n / 4 + 255) / 256;
  const unsigned blocks = (unsigned)std::min<size_t>(std::max<size_t>(want, 1), 2048);
  MOE_LAUNCH(k_add_f32, dim3(blocks), dim3(256), 0, s, out, y, n);
  return hipGetLastError();
}

// Word ranges gathered back to back into dst (the tiered layer copies its routing
// and x to the host in one transfer).
__global__ __launch_bounds__(256) void k_pack_words(PackWords p, uint32_t* __restrict__ dst) {
  uint32_t total = 0;
  for (int s = 0; s < PackWords::kMax; ++s) total += p.words[s];
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    uint32_t off = i;
    int s = 0;
    while (s < PackWords::kMax - 1 && off >= p.words[s]) off -= p.words[s++];
    dst[i] = p.src[s][off];
  }
}

hipError_t launch_pack_words(const PackWords& p, uint32_t* dst, hipStream_t s) {
  size_t total = 0;
  for (int i = 0; i < PackWords::kMax; ++i) total += p.words[i];
  if (total == 0) return hipSuccess;
  if (total > 0xFFFFFFFFu) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 1024);
  MOE_LAUNCH(k_pack_words, dim3(blocks), dim3(256), 0, s, p, dst);
  return hipGetLastError();
}

}  // namespace moe

// Router logits and top-k selection.
//
// Routing as the pages describe it: each token goes to 10 of a layer's 512
// experts (page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU",
// sections "What it is" and "How a 125B model fits in 12 GB").  The selection
// rule (largest logits, ties to the lower index) and the gates (softmax over the
// selected logits = full softmax renormalised over the k) are this library's
// reading of what the pages leave open.
#include <math.h>

#include "device.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router GEMV for small token counts: one wave per expert row; every lane reads
// 16-byte chunks of the bf16 row (coalesced 1 KB per wave instruction) and the
// same chunks of TB token rows, accumulating bf16 pair products in fp32
// (v_dot2c_f32_bf16, exact products), then a fixed-order wave reduction.
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, int T,
                                                     const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ bias, int E, int H,
                                                     float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const uint4* __restrict__ wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const int nch = H / 8;
  const float b = bias ? bias[e] : 0.0f;
  for (int t0 = 0; t0 < T; t0 += TB) {
    float acc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) acc[i] = 0.0f;
    for (int c = lane; c < nch; c += 64) {
      const uint4 w = wrow[c];
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (t0 + i < T) {
          const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)(t0 + i) * H)[c];
          float a = acc[i];
          a = dot2_bf16(w.x, xv.x, a);
          a = dot2_bf16(w.y, xv.y, a);
          a = dot2_bf16(w.z, xv.z, a);
          a = dot2_bf16(w.w, xv.w, a);
          acc[i] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const float s = wave_sum(acc[i]);
      if (lane == 0 && t0 + i < T) logits[(size_t)(t0 + i) * E + e] = s + b;
    }
  }
}

hipError_t launch_router_gemv(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s) {
  dim3 grid((E + 3) / 4);
  if (T <= 1)
    hipLaunchKernelGGL(k_router_gemv<1>, grid, dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  else if (T <= 4)
    hipLaunchKernelGGL(k_router_gemv<4>, grid, dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  else
    hipLaunchKernelGGL(k_router_gemv<8>, grid, dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Lane l holds logits l, l + 64, ...; k + 1 rounds
// of a wave arg-max under the total order (logit descending, index ascending)
// pick the k experts in order and then the (k+1)-th logit for the margin.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates,
                                              float* __restrict__ margin) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[VPL];
  unsigned taken = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[(size_t)t * E + e] : -INFINITY;
  }
  float my_v = 0.0f;
  int my_e = 0;
  float last = 0.0f, next = -INFINITY;
  for (int r = 0; r <= k && r < E; ++r) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (r < k) {
      if (lane == r) {
        my_v = bv;
        my_e = be;
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      last = bv;
    } else {
      next = bv;
    }
  }
  const float top = __shfl(my_v, 0, 64);
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    gates[(size_t)t * k + lane] = ex / sum;
  }
  if (margin && lane == 0) margin[t] = (k < E) ? (last - next) : INFINITY;
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                       hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk<2>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk<8>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin);
  else
    hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin);
  return hipGetLastError();
}

}  // namespace moe

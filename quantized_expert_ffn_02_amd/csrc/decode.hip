// Decode front end: router logits, activation-table prep, top-k and the
// permutation of a small token batch (T*k + T <= 1024 entries: a decode step or
// an MTP verify batch of 1 + 3 tokens, page "Strata Runs 125B Qwen3.8-Flash-Next
// on a 12GB Gaming GPU", section "How a 125B model fits in 12 GB") in two
// launches.
//
// k_route_front: the first blocks compute the logits of 4 experts each (one
// wave per bf16 router row, the row's and the tokens' 16-byte chunks all loaded
// before any arithmetic); the remaining blocks build the activation pair table.
// k_route_select: one block runs top-k for every token (a wave per token) and a
// stable counting sort of the T*k (+T shared) entries into offsets, sorted rows,
// the inverse map and the GEMV work items.  (A single fused launch with a
// last-block ticket needs agent-scope release/acquire fences on every block,
// which cost more than the second launch.)
#include <math.h>

#include "device.h"
#include "internal.h"
#include "mx.h"
#include "table.h"
#include "topk.h"

namespace moe {

// logits of expert row e for tokens [t0, t0 + TB): the row's NC 16-byte chunks
// per lane and the matching x chunks of all TB tokens are loaded before any
// arithmetic (one memory round trip per call).  Loads past the row or past T
// read a clamped address (no branch around a load); their products are zeroed
// or not stored.  With norm_sq, x is the layer input before its RMSNorm: each
// token's chunks are scaled by its row_inv_rms and rounded to bf16 first.
template <int TB, int NC>
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x, int T, int t0,
                                           const uint16_t* __restrict__ wr, float b, int E, int H, int e,
                                           float* __restrict__ logits, const float* __restrict__ norm_sq = nullptr,
                                           float eps = 0.0f) {
  const int lane = threadIdx.x & 63;
  const uint4* __restrict__ wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const int nch = H / 8;
  uint4 w[NC], xv[TB][NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = min(lane + 64 * u, nch - 1);
    w[u] = wrow[c];
#pragma unroll
    for (int i = 0; i < TB; ++i) xv[i][u] = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + i, T - 1) * H)[c];
  }
#pragma unroll
  for (int u = 0; u < NC; ++u)
    if (lane + 64 * u >= nch) w[u] = make_uint4(0u, 0u, 0u, 0u);
  if (norm_sq) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const float inv = row_inv_rms(norm_sq, min(t0 + i, T - 1), H, eps);
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        xv[i][u].x = bf16x2_scale(xv[i][u].x, inv);
        xv[i][u].y = bf16x2_scale(xv[i][u].y, inv);
        xv[i][u].z = bf16x2_scale(xv[i][u].z, inv);
        xv[i][u].w = bf16x2_scale(xv[i][u].w, inv);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      a = dot2_bf16(w[u].x, xv[i][u].x, a);
      a = dot2_bf16(w[u].y, xv[i][u].y, a);
      a = dot2_bf16(w[u].z, xv[i][u].z, a);
      a = dot2_bf16(w[u].w, xv[i][u].w, a);
    }
    const float sum = wave_sum_rows(a);
    if (lane == 0 && t0 + i < T) logits[(size_t)(t0 + i) * E + e] = sum + b;
  }
}

// all tokens, 4 at a time, for H <= 64 * 8 * NC
template <int NC>
__device__ __forceinline__ void router_row_all(const uint16_t* __restrict__ x, int T,
                                               const uint16_t* __restrict__ wr, float b, int E, int H, int e,
                                               float* __restrict__ logits, const float* __restrict__ norm_sq,
                                               float eps) {
  for (int t0 = 0; t0 < T; t0 += 4) router_row<4, NC>(x, T, t0, wr, b, E, H, e, logits, norm_sq, eps);
}

__device__ __forceinline__ void router_row_dispatch(const uint16_t* __restrict__ x, int T,
                                                    const uint16_t* __restrict__ wr, float b, int E, int H, int e,
                                                    float* __restrict__ logits,
                                                    const float* __restrict__ norm_sq = nullptr, float eps = 0.0f) {
  if (H <= 2560)
    router_row_all<5>(x, T, wr, b, E, H, e, logits, norm_sq, eps);
  else
    router_row_all<8>(x, T, wr, b, E, H, e, logits, norm_sq, eps);
}

// Router GEMV for any T: one wave per expert row, tokens 4 at a time.
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, int T,
                                                     const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ bias, int E, int H,
                                                     float* __restrict__ logits) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float b = bias ? bias[e] : 0.0f;
  router_row_dispatch(x, T, wr, b, E, H, e, logits);
}

hipError_t launch_router_gemv(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s) {
  MOE_LAUNCH(k_router_gemv, dim3((E + 3) / 4), dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  return hipGetLastError();
}

// The first (E + 3) / 4 blocks compute router rows; the blocks after them build
// the activation table, so its loads run alongside the router's instead of
// after them.
__global__ __launch_bounds__(256) void k_route_front(SmallRouteArgs a) {
  const int tid = threadIdx.x, wv = tid >> 6;
  const int rblocks = (a.E + 3) / 4;
  if ((int)blockIdx.x < rblocks) {
    const int e = blockIdx.x * 4 + wv;
    if (e < a.E) {
      const float b = a.bias ? a.bias[e] : 0.0f;
      router_row_dispatch(a.x, a.T, a.wr, b, a.E, a.H, e, a.logits, a.norm_sq, a.norm_eps);
    }
    return;
  }
  if (a.xmx_data) {
    // fp8-piece table (256-column form, read by the gate/up kernel): one
    // element per thread, a half wave per 32-column block
    // (T H is a multiple of 64, so every wave is whole); thread of position p
    // reads the weight index at p
    const int items = a.T * a.H;
    const int tblocks = gridDim.x - rblocks;
    for (int base = (blockIdx.x - rblocks) * 256; base < items; base += tblocks * 256) {
      const int it = base + tid;
      if (it < items) {
        const int row = it / a.H, col = it - row * a.H;   // a wave's 64 elements lie in one row
        const int B = col >> 5, p = col & 31;
        float v = bf16_to_f32(a.x[(size_t)row * a.H + 32 * B + mx_weight_at(p)]);
        if (a.norm_sq) v = (float)(__bf16)(v * row_inv_rms(a.norm_sq, row, a.H, a.norm_eps));
        mx_emit(v, row, mx_slot256(B), p, a.H, a.xmx_data, a.xmx_exps);
      }
    }
    return;
  }
  if (a.xpairs) {
    const int nblk = a.H / 32;
    const int items = a.T * nblk * 16;
    const int tblocks = gridDim.x - rblocks;
    for (int it = (blockIdx.x - rblocks) * 256 + tid; it < items; it += tblocks * 256) {
      const int row = it / (nblk * 16), rem = it % (nblk * 16);
      prep_x_item(a.x, row, a.H, rem >> 4, (rem >> 3) & 1, rem & 7, a.q3 != 0, a.xpairs, a.xinit);
    }
  }
}

static int route_front_blocks(const SmallRouteArgs& a) {
  const int rblocks = (a.E + 3) / 4;
  if (!a.xpairs && !a.xmx_data) return rblocks;
  const int items = a.xmx_data ? a.T * a.H : a.T * (a.H / 32) * 16;
  const int tblocks = (items + 255) / 256;
  return rblocks + (tblocks < 64 ? tblocks : 64);
}

template <int VPL>
__global__ __launch_bounds__(256) void k_route_select(SmallRouteArgs a) {
  __shared__ int s_cnt[1024];
  __shared__ int s_grp[1024 + 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // ---- phase 2: top-k, one wave per token
  const int k = a.k, T = a.T, E = a.E;
  for (int t = wv; t < T; t += 4)
    wave_topk_row<VPL>(a.logits + (size_t)t * E, E, k, a.ids + (size_t)t * k, a.gates + (size_t)t * k,
                       a.margin ? a.margin + t : nullptr, s_grp + t * k);
  // ---- phase 3: stable counting sort of n entries over G = E + 1 groups
  const int G = E + 1;
  const int n = T * k + (a.with_shared ? T : 0);
  for (int g = tid; g < 1024; g += 256) s_cnt[g] = 0;
  for (int r = T * k + tid; r < n; r += 256) s_grp[r] = E;
  __syncthreads();
  for (int r = tid; r < n; r += 256) atomicAdd(&s_cnt[s_grp[r]], 1);
  __syncthreads();
  // exclusive scans over the groups (each thread owns 4 consecutive groups) of
  // the entry counts and of the work-item counts ceil(count / items_per)
  const int IP = a.items_per;
  int c4[4], loc = 0, nzi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c4[i] = s_cnt[tid * 4 + i];
    loc += c4[i];
    nzi += (c4[i] + IP - 1) / IP;
  }
  int inc = loc, inci = nzi;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64), oi = __shfl_up(inci, off, 64);
    if (lane >= off) {
      inc += o;
      inci += oi;
    }
  }
  __shared__ int s_w[4], s_wi[4];
  if (lane == 63) {
    s_w[wv] = inc;
    s_wi[wv] = inci;
  }
  __syncthreads();
  int base = 0, basei = 0, tot = 0, toti = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < wv) {
      base += s_w[i];
      basei += s_wi[i];
    }
    tot += s_w[i];
    toti += s_wi[i];
  }
  int run = base + inc - loc, runi = basei + inci - nzi;
  __syncthreads();   // everyone has read s_cnt; reuse it for the offsets
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = tid * 4 + i;
    if (g < G) {
      a.offsets[g] = run;
      s_cnt[g] = run;
      for (int q = 0; q < c4[i]; q += IP) {
        a.items[3 * runi + 0] = g;
        a.items[3 * runi + 1] = run + q;
        a.items[3 * runi + 2] = min(IP, c4[i] - q);
        ++runi;
      }
    }
    run += c4[i];
  }
  if (tid == 0) {
    a.offsets[G] = tot;
    *a.n_items = toti;
  }
  __syncthreads();
  // stable position: offset of the group + number of earlier entries in it
  for (int r = tid; r < n; r += 256) {
    const int g = s_grp[r];
    int rank = 0;
    for (int q = 0; q < r; ++q) rank += s_grp[q] == g;
    const int pos = s_cnt[g] + rank;
    a.sorted_rows[pos] = r;
    a.row_to_sorted[r] = pos;
  }
}

hipError_t launch_route_front(const SmallRouteArgs& a, hipStream_t s) {
  MOE_LAUNCH(k_route_front, dim3(route_front_blocks(a)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route_small(const SmallRouteArgs& a, hipStream_t s) {
  MOE_LAUNCH(k_route_front, dim3(route_front_blocks(a)), dim3(256), 0, s, a);
  if (a.E <= 64)
    MOE_LAUNCH(k_route_select<1>, dim3(1), dim3(256), 0, s, a);
  else if (a.E <= 128)
    MOE_LAUNCH(k_route_select<2>, dim3(1), dim3(256), 0, s, a);
  else if (a.E <= 256)
    MOE_LAUNCH(k_route_select<4>, dim3(1), dim3(256), 0, s, a);
  else if (a.E <= 512)
    MOE_LAUNCH(k_route_select<8>, dim3(1), dim3(256), 0, s, a);
  else
    MOE_LAUNCH(k_route_select<16>, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

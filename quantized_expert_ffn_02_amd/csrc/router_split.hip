// Router logits of a batch between a decode step and a prompt chunk
// (16 < T < 1,024 tokens: an MTP verify batch of many sequences).
//
// logits[t, e] = x_t . Wr[e] (+ b[e]): bf16 operands, exact products, fp32
// accumulation (v_mfma_f32_32x32x16_bf16).  At these sizes the 128 x 128 tile
// kernel has a handful of blocks that each walk K = 2,560 serially, bound by
// memory latency.  Here a block takes 32 tokens x 64 experts and its W waves
// split K: wave w owns K steps [w UPW, (w + 1) UPW) of 64, loads its A (x) and B
// (router rows) fragments straight into registers two steps ahead of use, and
// runs 2 MFMAs per 16 K; the W partial tiles are summed in LDS in wave order
// (deterministic) and written with the bias.  Blocks walk the (token chunk,
// expert tile) space grid-stride, expert tile fastest.
#include <math.h>

#include "device.h"
#include "internal.h"
#include "mfma.h"

namespace moe {

struct RouterArgs {
  const uint16_t* x;     // bf16 [T][H]
  const uint16_t* wr;    // bf16 [E][H]
  const float* bias;     // fp32 [E] or NULL
  float* logits;         // fp32 [T][E]
  int T, E, H;
};

template <int W, int UPW>
__global__ __launch_bounds__(W * 64) void k_router_split(RouterArgs a) {
  __shared__ float red[W][16][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.H, nch = K / 64;
  const int ncol = (a.E + 63) / 64;
  const int units = ((a.T + 31) / 32) * ncol;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;

  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int chunk = unit / ncol, j = unit - chunk * ncol;
    const int m0 = chunk * 32, rows = min(32, a.T - m0);
    // token of this lane's A rows (rows past the chunk repeat its first token)
    const int rr = r32 < rows ? r32 : 0;
    const u32x4* __restrict__ ap = reinterpret_cast<const u32x4*>(a.x + (size_t)(m0 + rr) * K + kh);
    const int e0 = 64 * j + r32, e1 = e0 + 32;
    const u32x4* __restrict__ w0 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e0, a.E - 1) * K + kh);
    const u32x4* __restrict__ w1 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e1, a.E - 1) * K + kh);

    f16x_t acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;

    // registers of the wave's UPW steps; loads issued two steps ahead of use
    u32x4 A[UPW][4], B[UPW][8];
    auto issue = [&](int u) {
      const int step = min(wv * UPW + u, nch - 1);   // past the end: reload the last step, result unused
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        A[u][s] = ap[step * 8 + 2 * s];
        B[u][s] = w0[step * 8 + 2 * s];
        B[u][4 + s] = w1[step * 8 + 2 * s];
      }
    };
    auto compute = [&](int u) {
      if (wv * UPW + u >= nch) return;   // wave-uniform
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const b8_t fa = __builtin_bit_cast(b8_t, A[u][s]);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, B[u][s]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, B[u][4 + s]), acc1, 0, 0, 0);
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
      const int c0 = 64 * j + col, c1 = c0 + 32;
      float* lr = a.logits + (size_t)(m0 + row) * a.E;
      if (c0 < a.E) lr[c0] = v0[q] + (a.bias ? a.bias[c0] : 0.0f);
      if (c1 < a.E) lr[c1] = v1[q] + (a.bias ? a.bias[c1] : 0.0f);
    }
    __syncthreads();   // red is reused by the next unit
  }
}

hipError_t launch_router_split(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                               float* logits, hipStream_t s) {
  RouterArgs a;
  a.x = x;
  a.wr = wr;
  a.bias = bias;
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.H = H;
  const int units = ((T + 31) / 32) * ((E + 63) / 64);
  if (units <= 0) return hipSuccess;
  constexpr int W = 8;
  const int nch = H / 64;
  if (nch <= 2 * W)
    MOE_LAUNCH((k_router_split<W, 2>), dim3(units), dim3(W * 64), 0, s, a);
  else if (nch <= 5 * W)
    MOE_LAUNCH((k_router_split<W, 5>), dim3(units), dim3(W * 64), 0, s, a);
  else if (nch <= 8 * W)
    MOE_LAUNCH((k_router_split<W, 8>), dim3(units), dim3(W * 64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe

// Router logits of a batch between a decode step and a prompt chunk
// (16 < T < 1,024 tokens: an MTP verify batch of many sequences).
//
// logits[t, e] = x_t . Wr[e] (+ b[e]): bf16 operands, exact products, fp32
// accumulation (v_mfma_f32_32x32x16_bf16).  A unit is 32 tokens x 64 experts;
// at these sizes there are only (T / 32) x (E / 64) units, so K is also split
// over KS blocks (router_parts) to put a block on every compute unit.  Block
// (unit, ks) covers K range ks of KS; its 4 waves each take a quarter of that
// range, load all their A (x) and B (router rows) fragments at once, run 2
// MFMAs per 16 K, and the 4 partial tiles are summed in LDS in wave order.
// With KS = 1 the block adds the bias and writes the logits; otherwise it
// writes its partial sum to parts[ks] and the top-k kernel adds the KS parts
// in ks order and then the bias (route.hip), so the result is deterministic.
#include <math.h>

#include "device.h"
#include "internal.h"
#include "mfma.h"

namespace moe {

struct RouterArgs {
  const uint16_t* x;     // bf16 [T][H]
  const uint16_t* wr;    // bf16 [E][H]
  const float* bias;     // fp32 [E] or NULL
  float* out;            // KS = 1: logits [T][E]; else parts [KS][T][E]
  int T, E, H, KS;
};

// A wave's K range is REPS x NK 16-K fragments; each group of NK is loaded at
// once and then multiplied.
template <int NK>
__global__ __launch_bounds__(256) void k_router_split(RouterArgs a, int reps) {
  __shared__ float red[4][2][16][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.H;
  const int ncol = (a.E + 63) / 64;
  const int unit = blockIdx.x / a.KS, ks = blockIdx.x - unit * a.KS;
  const int chunk = unit / ncol, j = unit - chunk * ncol;
  const int m0 = chunk * 32, rows = min(32, a.T - m0);
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  // this wave's K range: [k0, k0 + 16 NK reps)
  const int k0 = (ks * 4 + wv) * 16 * NK * reps;
  const int rr = r32 < rows ? r32 : 0;   // rows past the chunk repeat its first token
  const u32x4* __restrict__ ap = reinterpret_cast<const u32x4*>(a.x + (size_t)(m0 + rr) * K + k0 + kh);
  const int e0 = 64 * j + r32, e1 = e0 + 32;
  const u32x4* __restrict__ w0 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e0, a.E - 1) * K + k0 + kh);
  const u32x4* __restrict__ w1 = reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e1, a.E - 1) * K + k0 + kh);
  f16x_t acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
  for (int g = 0; g < reps; ++g) {
    u32x4 A[NK], B0[NK], B1[NK];
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      A[u] = ap[2 * (g * NK + u)];
      B0[u] = w0[2 * (g * NK + u)];
      B1[u] = w1[2 * (g * NK + u)];
    }
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const b8_t fa = __builtin_bit_cast(b8_t, A[u]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, B0[u]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(b8_t, B1[u]), acc1, 0, 0, 0);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    red[wv][0][r][lane] = acc0[r];
    red[wv][1][r][lane] = acc1[r];
  }
  __syncthreads();
  // 2 x 16 x 64 outputs over 256 threads: 8 each, summed over the waves in order
  // The bias (KS = 1) is loaded before any store, and the stores take no
  // branch (an element outside the chunk's rows or past E gets an offset past
  // the plane's end, which the store drops): a store behind a branch that needs
  // a bias load made the compiler wait for every store in flight before it.
  const size_t plane = (size_t)a.T * a.E;
  float* __restrict__ dst = a.out + (a.KS > 1 ? (size_t)ks * plane : 0);
  const __amdgpu_buffer_rsrc_t dr = buffer_rsrc(dst, (uint32_t)plane * 4u);
  float bv[2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
    bv[f] = a.KS == 1 && a.bias ? a.bias[min(64 * j + 32 * f + (lane & 31), a.E - 1)] : 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int o = q * 256 + (int)threadIdx.x;   // o = f * 1024 + r * 64 + l, l = lane
    const int f = o >> 10, r = (o >> 6) & 15, l = o & 63;
    const float sum = ((red[0][f][r][l] + red[1][f][r][l]) + red[2][f][r][l]) + red[3][f][r][l];
    const int row = acc_row(r, l), col = 64 * j + 32 * f + (l & 31);
    const uint32_t off =
        row < rows && col < a.E ? ((uint32_t)(m0 + row) * (uint32_t)a.E + (uint32_t)col) * 4u : 0xFFFFFFF0u;
    const float v = a.KS > 1 ? sum : sum + bv[f];
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), dr, off, 0, 0);
  }
}

// K-split factor of the router for T tokens: enough blocks to cover the
// compute units, with every wave's quarter of a block's K a whole number of
// 16-K fragments (at most 8 parts).
int router_parts(int T, int E, int H) {
  if (T <= 16 || T >= 1024) return 1;
  const int units = ((T + 31) / 32) * ((E + 63) / 64);
  int ks = 1;
  while (ks < 8 && units * ks < 256 && (H / 16) % (8 * ks) == 0) ks *= 2;
  return ks;
}

hipError_t launch_router_split(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                               float* out, int parts, hipStream_t s) {
  RouterArgs a;
  a.x = x;
  a.wr = wr;
  a.bias = bias;
  a.out = out;
  a.T = T;
  a.E = E;
  a.H = H;
  a.KS = parts;
  const int units = ((T + 31) / 32) * ((E + 63) / 64);
  if (units <= 0) return hipSuccess;
  if (parts < 1 || (H / 16) % (4 * parts)) return hipErrorInvalidValue;
  const int nkw = H / 16 / (4 * parts);   // 16-K fragments per wave
  dim3 grid(units * parts);
  if (nkw % 10 == 0)
    MOE_LAUNCH(k_router_split<10>, grid, dim3(256), 0, s, a, nkw / 10);
  else if (nkw % 8 == 0)
    MOE_LAUNCH(k_router_split<8>, grid, dim3(256), 0, s, a, nkw / 8);
  else if (nkw % 5 == 0)
    MOE_LAUNCH(k_router_split<5>, grid, dim3(256), 0, s, a, nkw / 5);
  else if (nkw % 4 == 0)
    MOE_LAUNCH(k_router_split<4>, grid, dim3(256), 0, s, a, nkw / 4);
  else if (nkw % 2 == 0)
    MOE_LAUNCH(k_router_split<2>, grid, dim3(256), 0, s, a, nkw / 2);
  else
    MOE_LAUNCH(k_router_split<1>, grid, dim3(256), 0, s, a, nkw);
  return hipGetLastError();
}

}  // namespace moe

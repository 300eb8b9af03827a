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
#include "mx.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k for any T: one wave per token (topk.h).
// ---------------------------------------------------------------------------
// parts > 1: the logits are `parts` partial planes of [T][E] plus bias (the
// K-split router of router_split.hip), added here in plane order.
// With f16.x set, blocks of the same launch write the grouped GEMMs' activation
// copy of the rows (wave_row_to_f16, one wave per token, beside the token's
// selection), which then needs no launch of its own.
struct RowF16 {
  const uint16_t* x = nullptr;   // bf16 [T][H]
  int H = 0;                     // H % 16 == 0, H <= kRowF16MaxH
  uint16_t* out = nullptr;       // fp16 [T][H], pair order, scaled by 2^a
  int32_t* xexp = nullptr;       // a per row
};

// x' = x 2^a of one bf16 row by one wave, as k_x_to_f16_rows makes it (same
// bits): the largest magnitude from the bit patterns, a = bf16_row_exponent,
// then fp16 of x 2^a in pair order (u32 j of a 16-column group = columns j and
// j + 8).  Lane L takes the 16-column groups L, L + 64, L + 128.
__device__ __forceinline__ void wave_row_to_f16(const uint16_t* __restrict__ xr, int H, uint16_t* __restrict__ out,
                                                int32_t* __restrict__ xexp) {
  const int lane = threadIdx.x & 63, n16 = H / 16;
  const uint4* src = reinterpret_cast<const uint4*>(xr);
  uint4 v[3][2];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int g = lane + 64 * j;
    if (g < n16) {
      v[j][0] = src[2 * g];
      v[j][1] = src[2 * g + 1];
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    if (lane + 64 * j < n16) {
      const uint32_t in[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w, v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, max(in[i] & 0x7FFFu, (in[i] >> 16) & 0x7FFFu));
    }
  }
  const int a = bf16_row_exponent(wave_max_u32(m));
  if (lane == 0) *xexp = a;
  uint4* dst = reinterpret_cast<uint4*>(out);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int g = lane + 64 * j;
    if (g < n16) {
      const uint32_t in[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w, v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // column i (low half of in[i/2] if i even) and column i + 8
        const uint32_t v0 = (i & 1) ? (in[i >> 1] >> 16) : (in[i >> 1] & 0xFFFFu);
        const uint32_t v1 = (i & 1) ? (in[4 + (i >> 1)] >> 16) : (in[4 + (i >> 1)] & 0xFFFFu);
        const _Float16 f0 = (_Float16)ldexpf(bf16_to_f32(v0), a), f1 = (_Float16)ldexpf(bf16_to_f32(v1), a);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, f0) | ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
      }
      dst[2 * g] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[2 * g + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

// With tab.data set, blocks past the top-k's build x's fp8-piece table (mx.h,
// 256-column form) for the grouped GEMM's fp8 x fp4 tiles, on the compute units
// that the one-wave-per-token top-k leaves idle.
struct MxTab {
  const uint16_t* x = nullptr;   // bf16 [T][H], H % 256 == 0
  int H = 0;
  uint8_t* data = nullptr;
  uint8_t* exps = nullptr;
};

template <int VPL, bool PARTS>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates,
                                              float* __restrict__ margin, int parts, const float* __restrict__ bias,
                                              RowF16 f16, MxTab tab) {
  const int kb = (T + 3) / 4;                       // top-k blocks, then as many conversion blocks
  const int cb = f16.x ? 2 * kb : kb;
  const int b = blockIdx.x;
  if (b >= cb) {
    mx_table_pass(tab.x, T, tab.H, tab.data, tab.exps, b - cb, (int)gridDim.x - cb);
    return;
  }
  const int t = (b < kb ? b : b - kb) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (b >= kb) {
    wave_row_to_f16(f16.x + (size_t)t * f16.H, f16.H, f16.out + (size_t)t * f16.H, f16.xexp + t);
    return;
  }
  wave_topk_row<VPL, PARTS>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k,
                            margin ? margin + t : nullptr, nullptr, parts, (size_t)T * E, bias);
}

template <bool PARTS>
static hipError_t launch_topk_t(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                                int parts, const float* bias, const RowF16& f, const MxTab& mt, hipStream_t s) {
  dim3 grid((T + 3) / 4 * (f.x ? 2 : 1) + (mt.data ? mx_table_blocks(T, mt.H, 512) : 0));
  if (E <= 64)
    MOE_LAUNCH((k_topk<1, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias, f, mt);
  else if (E <= 128)
    MOE_LAUNCH((k_topk<2, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias, f, mt);
  else if (E <= 256)
    MOE_LAUNCH((k_topk<4, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias, f, mt);
  else if (E <= 512)
    MOE_LAUNCH((k_topk<8, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias, f, mt);
  else
    MOE_LAUNCH((k_topk<16, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias, f, mt);
  return hipGetLastError();
}

bool topk_row_f16_ok(int H) { return H % 16 == 0 && H <= kRowF16MaxH; }

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, int parts, const float* bias, const uint16_t* x, int H, uint16_t* xf16,
                       int32_t* xexp, const uint16_t* xt, uint8_t* xmx_data, uint8_t* xmx_exps) {
  RowF16 f;
  if (x) {
    if (!topk_row_f16_ok(H) || !xf16 || !xexp) return hipErrorInvalidValue;
    f.x = x;
    f.H = H;
    f.out = xf16;
    f.xexp = xexp;
  }
  MxTab mt;
  if (xmx_data) {
    if (!xt || !xmx_exps || H % 256) return hipErrorInvalidValue;
    mt.x = xt;
    mt.H = H;
    mt.data = xmx_data;
    mt.exps = xmx_exps;
  }
  if (parts > 1) return launch_topk_t<true>(logits, T, E, k, ids, gates, margin, parts, bias, f, mt, s);
  return launch_topk_t<false>(logits, T, E, k, ids, gates, margin, 1, nullptr, f, mt, s);
}

}  // namespace moe

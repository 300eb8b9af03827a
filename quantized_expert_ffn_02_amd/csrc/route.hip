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
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k for any T: one wave per token (topk.h).
// ---------------------------------------------------------------------------
// parts > 1: the logits are `parts` partial planes of [T][E] plus bias (the
// K-split router of router_split.hip), added here in plane order.
template <int VPL, bool PARTS>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates,
                                              float* __restrict__ margin, int parts, const float* __restrict__ bias) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk_row<VPL, PARTS>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k,
                            margin ? margin + t : nullptr, nullptr, parts, (size_t)T * E, bias);
}

template <bool PARTS>
static hipError_t launch_topk_t(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                                int parts, const float* bias, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64)
    MOE_LAUNCH((k_topk<1, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias);
  else if (E <= 128)
    MOE_LAUNCH((k_topk<2, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias);
  else if (E <= 256)
    MOE_LAUNCH((k_topk<4, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias);
  else if (E <= 512)
    MOE_LAUNCH((k_topk<8, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias);
  else
    MOE_LAUNCH((k_topk<16, PARTS>), grid, dim3(256), 0, s, logits, T, E, k, ids, gates, margin, parts, bias);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, int parts, const float* bias) {
  if (parts > 1) return launch_topk_t<true>(logits, T, E, k, ids, gates, margin, parts, bias, s);
  return launch_topk_t<false>(logits, T, E, k, ids, gates, margin, 1, nullptr, s);
}

}  // namespace moe

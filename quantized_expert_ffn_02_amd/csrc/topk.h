// Wave64 top-k selection over one token's router logits.
//
// Order: logit descending, expert index ascending (so exactly equal logits go to
// the lower index).  Each lane holds VPL logits (experts lane + 64 j), sorted once
// per lane; then k + 1 rounds of a wave arg-max over the lanes' heads pick the
// experts in order and the (k+1)-th logit for the margin.  The arg-max takes the
// 32-bit maximum of the heads' logit words with DPP moves (four steps inside
// each 16-lane row, two row broadcasts across rows, the result read from lane
// 63) and a ballot for its holder; only equal logits need a second maximum, over
// the index words.
#pragma once

#include <math.h>

#include "device.h"

namespace moe {

// Total order as one 64-bit key: order-preserving bits of the logit in the
// high word, the complement of the expert index in the low word, so the
// largest key is the largest logit with the lowest index.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float(ord ^ ((ord >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }

// Lanes without a source (or in rows outside ROW_MASK) read 0, the identity of
// an unsigned maximum, which lets the compiler fold the move into v_max_u32's
// DPP form.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
  return o > v ? o : v;
}

// Wave-uniform maximum of one 32-bit value per lane (the same DPP steps).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32_step<0xB1, 0xF>(v);
  v = dpp_max_u32_step<0x4E, 0xF>(v);
  v = dpp_max_u32_step<0x124, 0xF>(v);
  v = dpp_max_u32_step<0x128, 0xF>(v);
  v = dpp_max_u32_step<0x142, 0xA>(v);
  v = dpp_max_u32_step<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Keys of one token's top-k: lane r (< k) holds the key of rank r in ``mine``;
// ``last`` is the k-th key and ``next`` the (k+1)-th (0 when k == E).
struct TopkKeys {
  uint64_t mine, last, next;
};

// PARTS: the logits are the sum of np (<= 8) partial planes pstride floats
// apart (added in plane order) plus bias (if not NULL), as a K-split router
// leaves them.
// max_rounds < k + 1 stops after that many ranks (wave-uniform): lanes below it
// hold their ranks' keys, ``last`` and ``next`` are then not set.
template <int VPL, bool PARTS = false>
__device__ TopkKeys wave_topk_keys(const float* __restrict__ row, int E, int k, int np = 1, size_t pstride = 0,
                                   const float* __restrict__ bias = nullptr, int max_rounds = 0x7FFFFFFF) {
  const int lane = threadIdx.x & 63;
  // all VPL loads in flight at once (clamped index, no branch around a load)
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = row[min(lane + 64 * j, E - 1)];
  if constexpr (PARTS) {
    // planes 1 .. np - 1 (np <= 8), every load issued before the first add
    // (plane index clamped; clamped planes are not added)
    float w[7][VPL], bv[VPL];
#pragma unroll
    for (int p = 1; p < 8; ++p)
#pragma unroll
      for (int j = 0; j < VPL; ++j) w[p - 1][j] = row[(size_t)min(p, np - 1) * pstride + min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < VPL; ++j) bv[j] = bias ? bias[min(lane + 64 * j, E - 1)] : 0.0f;
#pragma unroll
    for (int p = 1; p < 8; ++p)
      if (p < np) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) v[j] += w[p - 1][j];
      }
    if (bias) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) v[j] += bv[j];
    }
  }
  uint64_t key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? topk_key(v[j], e) : 0ull;   // 0 sorts below every real key
  }
  // per-lane descending sort of the VPL keys
#pragma unroll
  for (int a = 1; a < VPL; ++a)
#pragma unroll
    for (int b = a; b > 0; --b)
      if (key[b] > key[b - 1]) {
        const uint64_t t = key[b];
        key[b] = key[b - 1];
        key[b - 1] = t;
      }
  // Each round: the wave maximum of the heads' logit words; a single holder
  // (the usual case) gives the key directly, equal logits fall back to the
  // maximum of their index words (the lowest expert index).
  uint32_t khi[VPL], klo[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    khi[j] = (uint32_t)(key[j] >> 32);
    klo[j] = (uint32_t)key[j];
  }
  TopkKeys r;
  r.mine = r.last = r.next = 0;
  const int rounds = min(k < E ? k + 1 : k, max_rounds);
  for (int q = 0; q < rounds; ++q) {
    const uint32_t mh = wave_max_u32(khi[0]);
    const uint64_t tied = __ballot(khi[0] == mh);
    uint32_t ml;
    if (__popcll(tied) == 1)
      ml = (uint32_t)__builtin_amdgcn_readlane((int)klo[0], (int)__builtin_ctzll(tied));
    else
      ml = wave_max_u32(khi[0] == mh ? klo[0] : 0u);
    const uint64_t best = ((uint64_t)mh << 32) | ml;
    if (q < k) {
      if (lane == q) r.mine = best;
      r.last = best;
      if (khi[0] == mh && klo[0] == ml) {   // the lane holding it pops its head
#pragma unroll
        for (int j = 0; j + 1 < VPL; ++j) {
          khi[j] = khi[j + 1];
          klo[j] = klo[j + 1];
        }
        khi[VPL - 1] = 0u;
        klo[VPL - 1] = 0u;
      }
    } else {
      r.next = best;
    }
  }
  return r;
}

// Expert id of rank i (wave-uniform).
__device__ __forceinline__ int topk_rank_id(const TopkKeys& r, int i) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)r.mine, i);
  return (int)~lo;
}

// ids[k], gates[k] (softmax of the selected logits = the full softmax
// renormalised over them) and the margin between rank k-1 and rank k.
__device__ __forceinline__ void topk_write(const TopkKeys& r, int E, int k, int32_t* __restrict__ ids_out,
                                           float* __restrict__ gates_out, float* __restrict__ margin_out,
                                           int32_t* __restrict__ ids_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const float my_v = key_value(r.mine);
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    const int my_e = key_index(r.mine);
    ids_out[lane] = my_e;
    gates_out[lane] = ex / sum;
    if (ids_lds) ids_lds[lane] = my_e;
  }
  if (margin_out && lane == 0) *margin_out = k < E ? key_value(r.last) - key_value(r.next) : INFINITY;
}

// Top-k of one token: logits row [E] -> ids[k], gates[k], margin.
template <int VPL, bool PARTS = false>
__device__ void wave_topk_row(const float* __restrict__ row, int E, int k, int32_t* __restrict__ ids_out,
                              float* __restrict__ gates_out, float* __restrict__ margin_out,
                              int32_t* __restrict__ ids_lds = nullptr, int np = 1, size_t pstride = 0,
                              const float* __restrict__ bias = nullptr) {
  const TopkKeys r = wave_topk_keys<VPL, PARTS>(row, E, k, np, pstride, bias);
  topk_write(r, E, k, ids_out, gates_out, margin_out, ids_lds);
}

}  // namespace moe

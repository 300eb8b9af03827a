// Expert FFN of a decode-sized batch (up to 16 tokens) without a permutation.
//
// A decode step or an MTP verify batch of 1 + 3 tokens (page "Strata Runs 125B
// Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "How a 125B model fits in
// 12 GB") has about as many distinct experts as entries, so sorting the entries
// by expert buys nothing: every entry r = t k + i (routed) or T k + t (shared)
// is addressed directly.  Three launches follow the router front end:
//
// k_decode_gateup: block (r, 64-row group).  Wave 0 selects the token's top-k
//   from the router logits (the block for rank 0 and row group 0 also writes
//   ids, gates and margin), then every wave streams its share of the chosen
//   expert's gate and up rows like the GEMV of gemv.hip, and the epilogue writes
//   h = SiLU(gate) * up straight into the down projection's pair table.
// k_decode_down: block (r, 64 output rows), K split over the waves; writes the
//   entry's output row already multiplied by its gate.
// k_decode_combine: out[t] = the token's gate-scaled routed rows in rank order,
//   then the shared expert's row, then the residual (fixed order), with an
//   optional bf16 copy.
#include <math.h>

#include "device.h"
#include "internal.h"
#include "table.h"
#include "topk.h"

namespace moe {

template <bool Q3, int W, int CPW, int VPL>
__global__ __launch_bounds__(W * 64) void k_decode_gateup(
    const uint8_t* __restrict__ r_codes, const uint8_t* __restrict__ r_hi, const uint16_t* __restrict__ r_scales,
    const uint8_t* __restrict__ s_codes, const uint8_t* __restrict__ s_hi, const uint16_t* __restrict__ s_scales,
    size_t code_stride, size_t hi_stride, size_t scale_stride, int K, int inter, int T, int k, int E,
    const float* __restrict__ logits, int32_t* __restrict__ ids_out, float* __restrict__ gates_out,
    float* __restrict__ margin_out, const uint32_t* __restrict__ tpairs, const float* __restrict__ tinit,
    uint32_t* __restrict__ down_pairs, float* __restrict__ down_init) {
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES;
  __shared__ float red[W][2][64];
  __shared__ int s_expert;
  const int r = blockIdx.x, rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Tk = T * k;
  int tok, grp;
  if (r < Tk) {
    tok = r / k;
    const int i = r - tok * k;
    if (wv == 0) {
      const TopkKeys keys = wave_topk_keys<VPL>(logits + (size_t)tok * E, E, k);
      if (lane == 0) s_expert = topk_rank_id(keys, i);
      if (i == 0 && rg == 0)
        topk_write(keys, E, k, ids_out + (size_t)tok * k, gates_out + (size_t)tok * k,
                   margin_out ? margin_out + tok : nullptr);
    }
    __syncthreads();
    grp = __builtin_amdgcn_readfirstlane(s_expert);
  } else {
    tok = r - Tk;
    grp = E;
  }
  const bool is_shared = grp == E;
  const size_t eidx = is_shared ? 0 : (size_t)grp;
  const uint4* __restrict__ codes =
      reinterpret_cast<const uint4*>((is_shared ? s_codes : r_codes) + eidx * code_stride);
  const uint32_t* __restrict__ scales =
      reinterpret_cast<const uint32_t*>((is_shared ? s_scales : r_scales) + eidx * scale_stride);
  const uint2* __restrict__ hib =
      Q3 ? reinterpret_cast<const uint2*>((is_shared ? s_hi : r_hi) + eidx * hi_stride) : nullptr;

  const int nch = K / 64, nblk = K / 32, n128 = K / 128;
  const int ng[2] = {rg, rg + inter / 64};   // gate rows, up rows
  const int c0 = wv * CPW;

  // all weight loads of this wave first
  uint4 w[2][CPW];
  uint32_t sc[2][CPW];
  uint2 hw[2][CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = c0 + u < nch ? c0 + u : nch - 1;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const size_t tile = (size_t)ng[m] * nch + c;
      w[m][u] = codes[tile * 64 + lane];
      sc[m][u] = scales[(((size_t)ng[m] * n128 + (c >> 1)) * 64 + lane) * 2 + (c & 1)];
      if (Q3) hw[m][u] = hib[tile * 64 + lane];
    }
  }
  const Q2Masks MQ = q2_masks();
  Q3Masks MH;
  if (Q3) MH = q3_masks();

  const uint32_t* __restrict__ xrow = tpairs + (size_t)tok * nblk * (SETS * 16);
  const float* __restrict__ irow = tinit + (size_t)tok * nblk;
  // straight-line over the CPW chunks: a chunk past the end of K (only when
  // W * CPW > K / 64) repeats the last chunk and its result is dropped
  float acc[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const bool valid = c0 + u < nch;
    const int c = valid ? c0 + u : nch - 1;
    const uint32_t* __restrict__ x0 = xrow + (size_t)(2 * c) * (SETS * 16);
    const uint32_t* __restrict__ x1 = x0 + SETS * 16;
    const float i0 = irow[2 * c], i1 = irow[2 * c + 1];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float a0 = q2_word_dot(w[m][u].x, x0, i0, MQ);
      a0 = q2_word_dot(w[m][u].y, x0 + 8, a0, MQ);
      float a1 = q2_word_dot(w[m][u].z, x1, i1, MQ);
      a1 = q2_word_dot(w[m][u].w, x1 + 8, a1, MQ);
      if (Q3) {
        a0 = q3_hi_dot(hw[m][u].x, x0 + 16, a0, MH);
        a0 = q3_hi_dot(hw[m][u].x >> 8, x0 + 24, a0, MH);
        a1 = q3_hi_dot(hw[m][u].y, x1 + 16, a1, MH);
        a1 = q3_hi_dot(hw[m][u].y >> 8, x1 + 24, a1, MH);
      }
      float t = fmaf(fp16_to_f32(sc[m][u] & 0xFFFFu), a0, acc[m]);
      t = fmaf(fp16_to_f32(sc[m][u] >> 16), a1, t);
      acc[m] = valid ? t : acc[m];
    }
  }
  red[wv][0][lane] = acc[0];
  red[wv][1][lane] = acc[1];
  __syncthreads();
  if (wv == 0) {
    float a = red[0][0][lane], b = red[0][1][lane];
    for (int u = 1; u < W; ++u) {
      a += red[u][0][lane];
      b += red[u][1][lane];
    }
    const float hv = a / (1.0f + expf(-a)) * b;
    emit_down_table<Q3>(hv, r, rg, inter, down_pairs, down_init);
  }
}

// Down projection of one entry r and 64 output rows, K split over W waves of
// CPW chunks; the epilogue scales by the entry's gate (1 for the shared expert)
// so that the combine only adds rows.
template <bool Q3, int W, int CPW>
__global__ __launch_bounds__(W * 64) void k_decode_down(
    const uint8_t* __restrict__ r_codes, const uint8_t* __restrict__ r_hi, const uint16_t* __restrict__ r_scales,
    const uint8_t* __restrict__ s_codes, const uint8_t* __restrict__ s_hi, const uint16_t* __restrict__ s_scales,
    size_t code_stride, size_t hi_stride, size_t scale_stride, int H, int K, int T, int k, int E,
    const int32_t* __restrict__ ids, const float* __restrict__ gates, const uint32_t* __restrict__ hpairs,
    const float* __restrict__ hinit, float* __restrict__ y) {
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * 2;   // hi and lo bf16 parts of h
  __shared__ float red[W][64];
  const int r = blockIdx.x, rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Tk = T * k;
  const int grp = r < Tk ? __builtin_amdgcn_readfirstlane(ids[r]) : E;
  const bool is_shared = grp == E;
  const size_t eidx = is_shared ? 0 : (size_t)grp;
  const uint4* __restrict__ codes =
      reinterpret_cast<const uint4*>((is_shared ? s_codes : r_codes) + eidx * code_stride);
  const uint32_t* __restrict__ scales =
      reinterpret_cast<const uint32_t*>((is_shared ? s_scales : r_scales) + eidx * scale_stride);
  const uint2* __restrict__ hib =
      Q3 ? reinterpret_cast<const uint2*>((is_shared ? s_hi : r_hi) + eidx * hi_stride) : nullptr;
  const int nch = K / 64, nblk = K / 32, n128 = K / 128;
  const int c0 = wv * CPW;

  uint4 w[CPW];
  uint32_t sc[CPW];
  uint2 hw[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = c0 + u < nch ? c0 + u : nch - 1;
    const size_t tile = (size_t)rg * nch + c;
    w[u] = codes[tile * 64 + lane];
    sc[u] = scales[(((size_t)rg * n128 + (c >> 1)) * 64 + lane) * 2 + (c & 1)];
    if (Q3) hw[u] = hib[tile * 64 + lane];
  }
  const Q2Masks MQ = q2_masks();
  Q3Masks MH;
  if (Q3) MH = q3_masks();

  const uint32_t* __restrict__ hrow = hpairs + (size_t)r * nblk * (SETS * 16);
  const float* __restrict__ irow = hinit + (size_t)r * nblk;
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const bool valid = c0 + u < nch;
    const int c = valid ? c0 + u : nch - 1;
    const uint32_t* __restrict__ xp = hrow + (size_t)(2 * c) * (SETS * 16);
    float a0 = irow[2 * c], a1 = irow[2 * c + 1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t* __restrict__ x0 = xp + (s * PLANES) * 16;
      const uint32_t* __restrict__ x1 = xp + SETS * 16 + (s * PLANES) * 16;
      a0 = q2_word_dot(w[u].x, x0, a0, MQ);
      a0 = q2_word_dot(w[u].y, x0 + 8, a0, MQ);
      a1 = q2_word_dot(w[u].z, x1, a1, MQ);
      a1 = q2_word_dot(w[u].w, x1 + 8, a1, MQ);
      if (Q3) {
        a0 = q3_hi_dot(hw[u].x, x0 + 16, a0, MH);
        a0 = q3_hi_dot(hw[u].x >> 8, x0 + 24, a0, MH);
        a1 = q3_hi_dot(hw[u].y, x1 + 16, a1, MH);
        a1 = q3_hi_dot(hw[u].y >> 8, x1 + 24, a1, MH);
      }
    }
    float t = fmaf(fp16_to_f32(sc[u] & 0xFFFFu), a0, acc);
    t = fmaf(fp16_to_f32(sc[u] >> 16), a1, t);
    acc = valid ? t : acc;
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    float a = red[0][lane];
    for (int u = 1; u < W; ++u) a += red[u][lane];
    const float g = r < Tk ? gates[r] : 1.0f;
    y[(size_t)r * H + rg * 64 + lane] = g * a;
  }
}

// out[t] = sum_{i<k} (g y)[t k + i] + y[T k + t] (+ residual[t]), fixed order;
// optional bf16 copy.  Four consecutive outputs per thread; the token's rows
// are loaded kBatch at a time before they are added (one memory round trip
// per batch, not per row).
__global__ __launch_bounds__(256) void k_decode_combine(const float* __restrict__ y, int T, int k, int H,
                                                        int with_shared, const uint16_t* __restrict__ residual,
                                                        float* __restrict__ out, uint16_t* __restrict__ out_bf16) {
  constexpr int kBatch = 12;
  const int t = blockIdx.y;
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q * 4 >= H) return;
  const size_t H4 = H / 4;
  const float4* __restrict__ y4 = reinterpret_cast<const float4*>(y);
  uint2 rb = make_uint2(0u, 0u);
  if (residual) rb = reinterpret_cast<const uint2*>(residual + (size_t)t * H)[q];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int n = k + (with_shared ? 1 : 0);
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j < n ? i0 + j : n - 1;
      const size_t r = i < k ? (size_t)t * k + i : (size_t)T * k + t;
      v[j] = y4[r * H4 + q];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (i0 + j < n) {
        acc.x += v[j].x;
        acc.y += v[j].y;
        acc.z += v[j].z;
        acc.w += v[j].w;
      }
    }
  }
  if (residual) {
    acc.x += bf16_to_f32(rb.x & 0xFFFFu);
    acc.y += bf16_to_f32(rb.x >> 16);
    acc.z += bf16_to_f32(rb.y & 0xFFFFu);
    acc.w += bf16_to_f32(rb.y >> 16);
  }
  reinterpret_cast<float4*>(out)[(size_t)t * H4 + q] = acc;
  if (out_bf16) {
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(out_bf16 + (size_t)t * H)[q] = o;
  }
}

bool decode_direct_ok(int T, int k, int with_shared, int H, int I) {
  return T >= 1 && T <= kDecodeDirectMaxTokens && H / 64 <= 64 && I / 64 <= 32;
}

template <bool Q3, int VPL>
static hipError_t launch_gateup_t(const DecodeFfnArgs& a, hipStream_t s) {
  const int nch = a.H / 64;
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  dim3 grid(entries, a.I / 64);
  const MatRef& r = a.r13;
  const MatRef& sh = a.s13;
#define MOE_DEC_ARGS                                                                                              \
  r.codes, r.hi, r.scales, sh.codes, sh.hi, sh.scales, r.code_stride, r.hi_stride, r.scale_stride, a.H, a.I, a.T, \
      a.k, a.E, a.logits, a.ids, a.gates, a.margin, a.xpairs, a.xinit, a.hpairs, a.hinit
  if (nch <= 8)
    MOE_LAUNCH((k_decode_gateup<Q3, 8, 1, VPL>), grid, dim3(512), 0, s, MOE_DEC_ARGS);
  else if (nch <= 16)
    MOE_LAUNCH((k_decode_gateup<Q3, 8, 2, VPL>), grid, dim3(512), 0, s, MOE_DEC_ARGS);
  else if (nch <= 40)
    MOE_LAUNCH((k_decode_gateup<Q3, 8, 5, VPL>), grid, dim3(512), 0, s, MOE_DEC_ARGS);
  else
    MOE_LAUNCH((k_decode_gateup<Q3, 16, 4, VPL>), grid, dim3(1024), 0, s, MOE_DEC_ARGS);
#undef MOE_DEC_ARGS
  return hipGetLastError();
}

hipError_t launch_decode_gateup(const DecodeFfnArgs& a, hipStream_t s) {
  if (a.q3) return a.E <= 512 ? launch_gateup_t<true, 8>(a, s) : launch_gateup_t<true, 16>(a, s);
  return a.E <= 512 ? launch_gateup_t<false, 8>(a, s) : launch_gateup_t<false, 16>(a, s);
}

// Down launch shapes: 10 waves x 1 chunk for a single token (more blocks in
// flight), 5 x 2 otherwise; K beyond 640 uses 8 waves of up to 4 chunks.
template <bool Q3>
static hipError_t launch_down_t(const DecodeFfnArgs& a, hipStream_t s) {
  const int nch = a.I / 64;
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  dim3 grid(entries, a.H / 64);
  const MatRef& r = a.r2;
  const MatRef& sh = a.s2;
#define MOE_DEC_ARGS                                                                                          \
  r.codes, r.hi, r.scales, sh.codes, sh.hi, sh.scales, r.code_stride, r.hi_stride, r.scale_stride, a.H, a.I, \
      a.T, a.k, a.E, a.ids, a.gates, a.hpairs, a.hinit, a.y
  if (nch <= 10 && a.T == 1)
    MOE_LAUNCH((k_decode_down<Q3, 10, 1>), grid, dim3(640), 0, s, MOE_DEC_ARGS);
  else if (nch <= 10)
    MOE_LAUNCH((k_decode_down<Q3, 5, 2>), grid, dim3(320), 0, s, MOE_DEC_ARGS);
  else
    MOE_LAUNCH((k_decode_down<Q3, 8, 4>), grid, dim3(512), 0, s, MOE_DEC_ARGS);
#undef MOE_DEC_ARGS
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeFfnArgs& a, hipStream_t s) {
  return a.q3 ? launch_down_t<true>(a, s) : launch_down_t<false>(a, s);
}

hipError_t launch_decode_combine(const DecodeFfnArgs& a, hipStream_t s) {
  dim3 grid((a.H / 4 + 255) / 256, a.T);
  MOE_LAUNCH(k_decode_combine, grid, dim3(256), 0, s, a.y, a.T, a.k, a.H, a.with_shared, a.residual, a.out,
                     a.out_bf16);
  return hipGetLastError();
}

}  // namespace moe

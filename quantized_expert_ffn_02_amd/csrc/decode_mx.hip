// Expert FFN of a decode-sized batch with 2-bit weights on the block-scaled
// fp8 x fp4 matrix cores (mx.h gives the number formats and operand layouts).
//
// Same launches and work split as the VALU kernels of decode_ffn.hip (entries
// addressed directly, page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB
// Gaming GPU", section "How a 125B model fits in 12 GB"):
//
// k_decode_gateup_mx: block (entry r, 64 rows of gate and of up).  Wave 0
//   selects the token's top-k from the router logits; every wave reads its
//   chunks of the token's activation table first (they do not depend on the
//   expert), then its 16-row x 128-column weight fragments of the chosen
//   expert, and runs one MFMA per fragment.  The partial sums of the waves and
//   blocks are added in a fixed order, and the epilogue writes
//   h = SiLU(gate) * up as the down projection's activation table.
// k_decode_down_mx: block (entry r, 64 NG output rows), the K = I columns split
//   over the waves; the epilogue scales by the entry's gate.
//
// The combine is k_decode_combine (decode_ffn.hip).
#include <math.h>

#include "device.h"
#include "internal.h"
#include "mfma.h"
#include "mx.h"
#include "topk.h"

namespace moe {

// Weight rows of one 64-row group ng of an expert matrix, decode layout: tile
// (ng, c64) of 64 rows x 64 columns is 1,024 bytes, row-major by row, 16 bytes
// per row (two 32-weight blocks of two u32 words); scales per (ng, 128-column
// chunk) are 64 rows x 4 fp16.
struct MxLanes {
  uint32_t code[4];    // byte offset of this lane's 8 code bytes, subgroup s (16 rows), chunk 0
  uint32_t scale[4];   // byte offset of its fp16 scale, subgroup s, chunk 0
};

__device__ __forceinline__ MxLanes mx_weight_lanes(int lane) {
  const int n = lane & 15, G = lane >> 4;
  MxLanes L;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    L.code[s] = (uint32_t)((((G >> 1) * 64 + 16 * s + n) * 16) + 8 * (G & 1));
    L.scale[s] = (uint32_t)(((16 * s + n) * 4 + G) * 2);
  }
  return L;
}

// Scalar offsets of row group ng and chunk c (K columns).
__device__ __forceinline__ uint32_t mx_code_soff(int ng, int c, int K) {
  return (uint32_t)(((size_t)ng * (K / 64) + 2 * c) * 1024);
}
__device__ __forceinline__ uint32_t mx_scale_soff(int ng, int c, int K) {
  return (uint32_t)(((size_t)ng * (K / 128) + c) * 512);
}

// Activation operand of chunk c and this lane's scale byte.
struct MxAct {
  u32x4 lo, hi;
  uint32_t sa;
};

__device__ __forceinline__ MxAct mx_load_act(__amdgpu_buffer_rsrc_t rd, __amdgpu_buffer_rsrc_t re, const MxALane& AL,
                                             int c) {
  MxAct A;
  A.lo = __builtin_amdgcn_raw_buffer_load_b128(rd, AL.off_lo, c * 128 * kMxPieces, 0);
  A.hi = __builtin_amdgcn_raw_buffer_load_b128(rd, AL.off_hi, c * 128 * kMxPieces, 0);
  A.sa = __builtin_amdgcn_raw_buffer_load_b8(re, AL.exp_off, c * 16, 0);
  return A;
}

__device__ __forceinline__ mx_v8i mx_act_operand(const MxAct& A) {
  mx_v8i a;
  a[0] = (int)A.lo.x;
  a[1] = (int)A.lo.y;
  a[2] = (int)A.lo.z;
  a[3] = (int)A.lo.w;
  a[4] = (int)A.hi.x;
  a[5] = (int)A.hi.y;
  a[6] = (int)A.hi.z;
  a[7] = (int)A.hi.w;
  return a;
}

// y + s * (sum of the four pieces' outputs) for this lane's (weight row, block).
__device__ __forceinline__ float mx_accumulate(const mx_v4f& o, uint32_t scale16, float y) {
  return fmaf(fp16_to_f32(scale16), (o[0] + o[1]) + (o[2] + o[3]), y);
}

// Gate/up in the 256-column form: per 256 columns and 16-row subgroup, lane
// (n, q) = (lane % 16, lane / 16) loads the 16 code bytes of row n, 64-column
// chunk q (blocks 2 q and 2 q + 1) and their two fp16 scales; the first MFMA
// takes the even blocks (words 0, 1), the second the odd ones (words 2, 3).
template <int W, int SPW, int VPL>
__global__ __launch_bounds__(W * 64) void k_decode_gateup_mx(MxFfnArgs a) {
  __shared__ float red[W][8][64];
  __shared__ int s_expert;
  const int r = blockIdx.x, rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.H, ns = K / 256;
  const int Tk = a.T * a.k;
  const int tok = r < Tk ? r / a.k : r - Tk;
  const int s0 = wv * SPW;

  // The token's activation chunks do not depend on the expert: waves that do
  // not select the top-k issue them first (wave 0 issues them after the
  // selection, so that its logit loads do not queue behind them).
  const MxALane AL = mx_a_lane(lane);
  const __amdgpu_buffer_rsrc_t rxd = buffer_rsrc(a.xdata + (size_t)tok * mx_data_bytes(K), (uint32_t)mx_data_bytes(K));
  const __amdgpu_buffer_rsrc_t rxe = buffer_rsrc(a.xexps + (size_t)tok * mx_exps_bytes(K), (uint32_t)mx_exps_bytes(K));
  MxAct X[SPW][2];
  auto load_x = [&]() {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) X[u][pi] = mx_load_act(rxd, rxe, AL, 2 * min(s0 + u, ns - 1) + pi);
  };
  const bool select = r < Tk;
  if (!select || wv != 0) load_x();

  int grp;
  if (select) {
    const int i = r - tok * a.k;
    if (wv == 0) {
      const TopkKeys keys = wave_topk_keys<VPL>(a.logits + (size_t)tok * a.E, a.E, a.k);
      if (lane == 0) s_expert = topk_rank_id(keys, i);
      if (i == 0 && rg == 0)
        topk_write(keys, a.E, a.k, a.ids + (size_t)tok * a.k, a.gates + (size_t)tok * a.k,
                   a.margin ? a.margin + tok : nullptr);
    }
    __syncthreads();
    grp = __builtin_amdgcn_readfirstlane(s_expert);
  } else {
    grp = a.E;
  }
  if (select && wv == 0) load_x();
  const bool is_shared = grp == a.E;
  const MatRef& M = is_shared ? a.s13 : a.r13;
  const size_t eidx = is_shared ? 0 : (size_t)grp;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(M.codes + eidx * M.code_stride, (uint32_t)M.code_stride);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(M.scales + eidx * M.scale_stride, (uint32_t)(M.scale_stride * 2));
  const int n = lane & 15, q = lane >> 4;
  const int ng[2] = {rg, rg + a.I / 64};   // gate rows, up rows
  const int nch64 = K / 64, n128 = K / 128;

  // every weight load of this wave, then the products
  u32x4 cw[SPW][2][4];
  uint32_t sc[SPW][2][4];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int c = min(s0 + u, ns - 1);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t cso = (uint32_t)(((size_t)ng[m] * nch64 + 4 * c) * 1024);
      const uint32_t sso = (uint32_t)(((size_t)ng[m] * n128 + 2 * c) * 512);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        cw[u][m][s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(q * 1024 + (16 * s + n) * 16), cso, 0);
        sc[u][m][s] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(((q >> 1) * 64 + 16 * s + n) * 8 + (q & 1) * 4), sso, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
  float y[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < 4; ++s) y[m][s] = 0.0f;
  const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const bool valid = s0 + u < ns;
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
      const mx_v8i A = mx_act_operand(X[u][pi]);
      const mx_v4f off = mx_mfma(A, mx_minus_one(), (int)X[u][pi].sa, zero);   // -2 sum v per (piece, block)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4& w = cw[u][m][s];
          const mx_v4f o = mx_mfma(A, pi ? mx_weights(w.z, w.w) : mx_weights(w.x, w.y), (int)X[u][pi].sa, off);
          const float t = mx_accumulate(o, pi ? sc[u][m][s] >> 16 : sc[u][m][s] & 0xFFFFu, y[m][s]);
          y[m][s] = valid ? t : y[m][s];
        }
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < 4; ++s) red[wv][m * 4 + s][lane] = y[m][s];
  __syncthreads();
  if (wv == 0) {
    // row lane of the 64: subgroup s = lane / 16, row n = lane % 16 of it;
    // waves in order, then the four lane groups in order
    const int s = lane >> 4, nn = lane & 15;
    float g = 0.0f, up = 0.0f;
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        g += red[w][s][16 * qq + nn];
        up += red[w][4 + s][16 * qq + nn];
      }
    const float hv = g / (1.0f + expf(-g)) * up;
    // h row lane of this block is column 64 rg + lane of the entry's h: block
    // 2 rg + lane / 32 (128-column table form, read by the down kernel),
    // weight index lane % 32
    mx_emit(hv, r, mx_slot128(2 * rg + (lane >> 5)), mx_pos_of_weight(lane & 31), a.I, a.hdata, a.hexps);
  }
}

// NG 64-row output groups per block; K = I columns over W waves of CPW chunks.
template <int W, int CPW, int NG>
__global__ __launch_bounds__(W * 64) void k_decode_down_mx(MxFfnArgs a) {
  __shared__ float red[W][4 * NG][64];
  const int r = blockIdx.x, rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.I, nc = K / 128;
  const int Tk = a.T * a.k;
  const int c0 = wv * CPW;

  const MxALane AL = mx_a_lane(lane);
  const __amdgpu_buffer_rsrc_t rhd = buffer_rsrc(a.hdata + (size_t)r * mx_data_bytes(K), (uint32_t)mx_data_bytes(K));
  const __amdgpu_buffer_rsrc_t rhe = buffer_rsrc(a.hexps + (size_t)r * mx_exps_bytes(K), (uint32_t)mx_exps_bytes(K));
  MxAct X[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) X[u] = mx_load_act(rhd, rhe, AL, min(c0 + u, nc - 1));

  const int grp = r < Tk ? __builtin_amdgcn_readfirstlane(a.ids[r]) : a.E;
  const bool is_shared = grp == a.E;
  const MatRef& M = is_shared ? a.s2 : a.r2;
  const size_t eidx = is_shared ? 0 : (size_t)grp;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(M.codes + eidx * M.code_stride, (uint32_t)M.code_stride);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(M.scales + eidx * M.scale_stride, (uint32_t)(M.scale_stride * 2));
  const MxLanes WL = mx_weight_lanes(lane);

  uint2 cw[CPW][NG][4];
  uint32_t sc[CPW][NG][4];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = min(c0 + u, nc - 1);
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) {
      const int ngr = rg * NG + gq;
      const uint32_t cso = mx_code_soff(ngr, c, K), sso = mx_scale_soff(ngr, c, K);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, WL.code[s], cso, 0);
        cw[u][gq][s] = make_uint2(v[0], v[1]);
        sc[u][gq][s] = __builtin_amdgcn_raw_buffer_load_b16(rs, WL.scale[s], sso, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
  float y[NG][4];
#pragma unroll
  for (int gq = 0; gq < NG; ++gq)
#pragma unroll
    for (int s = 0; s < 4; ++s) y[gq][s] = 0.0f;
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const bool valid = c0 + u < nc;
    const mx_v8i A = mx_act_operand(X[u]);
    const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const mx_v4f off = mx_mfma(A, mx_minus_one(), (int)X[u].sa, zero);   // -2 sum v per (piece, block)
#pragma unroll
    for (int gq = 0; gq < NG; ++gq)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const mx_v4f o = mx_mfma(A, mx_weights(cw[u][gq][s].x, cw[u][gq][s].y), (int)X[u].sa, off);
        const float t = mx_accumulate(o, sc[u][gq][s], y[gq][s]);
        y[gq][s] = valid ? t : y[gq][s];
      }
  }
#pragma unroll
  for (int gq = 0; gq < NG; ++gq)
#pragma unroll
    for (int s = 0; s < 4; ++s) red[wv][gq * 4 + s][lane] = y[gq][s];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 64 * NG) {
    const int gq = t >> 6, s = (t >> 4) & 3, n = t & 15;
    float acc = 0.0f;
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc += red[w][gq * 4 + s][16 * q + n];
    const float gate = r < Tk ? a.gates[r] : 1.0f;
    a.y[(size_t)r * a.H + (size_t)rg * 64 * NG + t] = gate * acc;
  }
}

bool decode_mx_ok(int H, int I, int q3) { return !q3 && H % 256 == 0 && I % 128 == 0 && H / 256 <= 20 && I / 128 <= 10; }

hipError_t launch_decode_gateup_mx(const MxFfnArgs& a, hipStream_t s) {
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  const int ns = a.H / 256;
  dim3 grid(entries, a.I / 64);
  if (ns <= 10) {
    if (a.E <= 512)
      MOE_LAUNCH((k_decode_gateup_mx<10, 1, 8>), grid, dim3(640), 0, s, a);
    else
      MOE_LAUNCH((k_decode_gateup_mx<10, 1, 16>), grid, dim3(640), 0, s, a);
  } else {
    if (a.E <= 512)
      MOE_LAUNCH((k_decode_gateup_mx<10, 2, 8>), grid, dim3(640), 0, s, a);
    else
      MOE_LAUNCH((k_decode_gateup_mx<10, 2, 16>), grid, dim3(640), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_down_mx(const MxFfnArgs& a, hipStream_t s) {
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  const int nc = a.I / 128;
  dim3 grid(entries, a.H / 64);
  if (nc <= 5)
    MOE_LAUNCH((k_decode_down_mx<5, 1, 1>), grid, dim3(320), 0, s, a);
  else
    MOE_LAUNCH((k_decode_down_mx<5, 2, 1>), grid, dim3(320), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

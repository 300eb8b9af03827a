// Expert FFN of a decode-sized batch with 2-bit weights on the block-scaled
// fp8 x fp4 matrix cores (mx.h gives the number formats and operand layouts).
//
// Same launches and work split as the VALU kernels of decode_ffn.hip (entries
// addressed directly, page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB
// Gaming GPU", section "How a 125B model fits in 12 GB"):
//
// k_decode_gateup_mx: block (entry r, 64 rows of gate and of up).  Wave 0
//   selects the token's top-k from the router logits; every wave reads its
//   chunks of the token's activation table (they do not depend on the
//   expert), then the chosen expert's 16-byte code lanes of its 256 columns
//   (two 32-weight blocks each, two MFMAs per load).  The partial sums of the
//   waves and lanes are added in a fixed order, and the epilogue writes
//   h = SiLU(gate) * up as the down projection's activation table.
// k_decode_down_mx: block (entry r, 64 output rows), one wave per 256 columns
//   of K = I and one for a 128-column tail; the epilogue scales by the
//   entry's gate.
//
// The combine is k_decode_combine (decode_ffn.hip).
#include <math.h>

#include <algorithm>

#include "device.h"
#include "internal.h"
#include "mfma.h"
#include "mx.h"
#include "topk.h"

namespace moe {

// Weight layout (decode form): rows in groups of 64; tile (group, 64-column
// chunk) is 1,024 bytes, 16 bytes per row (two 32-weight blocks of two u32
// words); scales per (group, 128-column chunk) are 64 rows x 4 fp16.

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

// Gate/up in the 256-column form: per 256 columns and 16-row subgroup, lane
// (n, q) = (lane % 16, lane / 16) loads the 16 code bytes of row n, 64-column
// chunk q (blocks 2 q and 2 q + 1) and their two fp16 scales; the first MFMA
// takes the even blocks (words 0, 1), the second the odd ones (words 2, 3).
template <int W, int SPW, int VPL, int RG = 64>
__global__ __launch_bounds__(W * 64) void k_decode_gateup_mx(MxFfnArgs a) {
  constexpr int NSG = RG / 16;   // 16-row subgroups of gate (and of up) per block
  __shared__ __attribute__((aligned(16))) float red[W][2 * NSG][64];
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
      // only the block that writes the token's ids, gates and margin needs all
      // k + 1 ranks; the others stop at their own
      const bool writer = i == 0 && rg == 0;
      const TopkKeys keys =
          wave_topk_keys<VPL>(a.logits + (size_t)tok * a.E, a.E, a.k, 1, 0, nullptr, writer ? 0x7FFFFFFF : i + 1);
      if (lane == 0) s_expert = topk_rank_id(keys, i);
      if (writer)
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
  // this block's RG gate rows (and up rows) start at row ro of 64-row group ng
  const int ng[2] = {(rg * RG) / 64, (rg * RG) / 64 + a.I / 64};   // gate rows, up rows
  const int ro = (rg * RG) % 64;
  const int nch64 = K / 64, n128 = K / 128;

  // every weight load of this wave, then the products
  u32x4 cw[SPW][2][NSG];
  uint32_t sc[SPW][2][NSG];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int c = min(s0 + u, ns - 1);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t cso = (uint32_t)(((size_t)ng[m] * nch64 + 4 * c) * 1024);
      const uint32_t sso = (uint32_t)(((size_t)ng[m] * n128 + 2 * c) * 512);
#pragma unroll
      for (int s = 0; s < NSG; ++s) {
        cw[u][m][s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(q * 1024 + (ro + 16 * s + n) * 16), cso, 0);
        sc[u][m][s] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(((q >> 1) * 64 + ro + 16 * s + n) * 8 + (q & 1) * 4), sso, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
  float y[2][NSG];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < NSG; ++s) y[m][s] = 0.0f;
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
        for (int s = 0; s < NSG; ++s) {
          const u32x4& w = cw[u][m][s];
          const mx_v4f o = mx_mfma(A, pi ? mx_weights(w.z, w.w) : mx_weights(w.x, w.y), (int)X[u][pi].sa, off);
          const float t = mx_accumulate(o, pi ? sc[u][m][s] >> 16 : sc[u][m][s] & 0xFFFFu, y[m][s]);
          y[m][s] = valid ? t : y[m][s];
        }
    }
  }
  // partial sums at [wave][m * 4 + s][row n][lane group q], so that each row's
  // four lane groups are one 16-byte read
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < NSG; ++s) red[wv][m * NSG + s][(lane & 15) * 4 + (lane >> 4)] = y[m][s];
  __syncthreads();
  if (wv == 0) {
    // row lane of the RG: subgroup s = lane / 16, row n = lane % 16 of it;
    // waves in order, then the four lane groups in order (lanes past RG
    // repeat rows and store nothing)
    const int s = (lane >> 4) & (NSG - 1), nn = lane & 15;
    float g = 0.0f, up = 0.0f;
    for (int w = 0; w < W; ++w) {
      const float4 gv = *reinterpret_cast<const float4*>(&red[w][s][nn * 4]);
      const float4 uv = *reinterpret_cast<const float4*>(&red[w][NSG + s][nn * 4]);
      g += gv.x;
      g += gv.y;
      g += gv.z;
      g += gv.w;
      up += uv.x;
      up += uv.y;
      up += uv.z;
      up += uv.w;
    }
    const float hv = g / (1.0f + expf(-g)) * up;
    // h row lane of this block is column RG rg + lane of the entry's h: block
    // (RG rg + lane) / 32 (mixed table form, read by the down kernel), weight
    // index lane % 32
    mx_emit(hv, r, mx_slot_mixed((rg * RG + lane) >> 5, a.I), mx_pos_of_weight(lane & 31), a.I, a.hdata, a.hexps,
            lane < RG);
  }
}

// Down projection of entry r and 64 output rows; K = I = 256 NS + 128 TAIL
// columns, one wave per 256 columns (16-byte code lanes, two MFMAs per load
// as in the gate/up kernel) and one for a 128-column tail (8-byte code lanes,
// one MFMA per load).  The epilogue scales by the entry's gate.
template <int NS, int TAIL>
__global__ __launch_bounds__((NS + TAIL) * 64) void k_decode_down_mx(MxFfnArgs a) {
  constexpr int W = NS + TAIL;
  __shared__ float red[W][4][64];
  const int r = blockIdx.x, rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.I;
  const int Tk = a.T * a.k;
  const bool tail = wv >= NS;   // wave-uniform

  const MxALane AL = mx_a_lane(lane);
  const __amdgpu_buffer_rsrc_t rhd = buffer_rsrc(a.hdata + (size_t)r * mx_data_bytes(K), (uint32_t)mx_data_bytes(K));
  const __amdgpu_buffer_rsrc_t rhe = buffer_rsrc(a.hexps + (size_t)r * mx_exps_bytes(K), (uint32_t)mx_exps_bytes(K));
  // virtual chunks: 2 wv (even blocks), 2 wv + 1 (odd blocks); the tail wave's 128 columns are chunk 2 NS
  MxAct X0 = mx_load_act(rhd, rhe, AL, tail ? 2 * NS : 2 * wv);
  MxAct X1 = mx_load_act(rhd, rhe, AL, tail ? 2 * NS : 2 * wv + 1);

  const int grp = r < Tk ? __builtin_amdgcn_readfirstlane(a.ids[r]) : a.E;
  const bool is_shared = grp == a.E;
  const MatRef& M = is_shared ? a.s2 : a.r2;
  const size_t eidx = is_shared ? 0 : (size_t)grp;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(M.codes + eidx * M.code_stride, (uint32_t)M.code_stride);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(M.scales + eidx * M.scale_stride, (uint32_t)(M.scale_stride * 2));
  const int n = lane & 15, q = lane >> 4;
  const int nch64 = K / 64, n128 = K / 128;

  u32x4 cw[4];
  uint32_t sc[4];
  if (!tail) {
    const uint32_t cso = (uint32_t)(((size_t)rg * nch64 + 4 * wv) * 1024);
    const uint32_t sso = (uint32_t)(((size_t)rg * n128 + 2 * wv) * 512);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cw[s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(q * 1024 + (16 * s + n) * 16), cso, 0);
      sc[s] = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(((q >> 1) * 64 + 16 * s + n) * 8 + (q & 1) * 4), sso, 0);
    }
  } else {
    // 128-column chunk c = 2 NS: lane (n, q) reads block q of row n (8 bytes) and its scale
    const int c = 2 * NS;
    const uint32_t cso = (uint32_t)(((size_t)rg * nch64 + 2 * c) * 1024);
    const uint32_t sso = (uint32_t)(((size_t)rg * n128 + c) * 512);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(
          rc, (uint32_t)((((q >> 1) * 64 + 16 * s + n) * 16) + 8 * (q & 1)), cso, 0);
      cw[s] = u32x4{v[0], v[1], 0u, 0u};
      sc[s] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)(((16 * s + n) * 4 + q) * 2), sso, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
  const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  {
    const mx_v8i A = mx_act_operand(X0);
    const mx_v4f off = mx_mfma(A, mx_minus_one(), (int)X0.sa, zero);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const mx_v4f o = mx_mfma(A, mx_weights(cw[s].x, cw[s].y), (int)X0.sa, off);
      y[s] = mx_accumulate(o, sc[s] & 0xFFFFu, y[s]);
    }
  }
  if (!tail) {
    const mx_v8i A = mx_act_operand(X1);
    const mx_v4f off = mx_mfma(A, mx_minus_one(), (int)X1.sa, zero);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const mx_v4f o = mx_mfma(A, mx_weights(cw[s].z, cw[s].w), (int)X1.sa, off);
      y[s] = mx_accumulate(o, sc[s] >> 16, y[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) red[wv][s][lane] = y[s];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 64) {
    const int s = t >> 4, nn = t & 15;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) acc += red[w][s][16 * qq + nn];
    const float gate = r < Tk ? a.gates[r] : 1.0f;
    a.y[(size_t)r * a.H + (size_t)rg * 64 + t] = gate * acc;
  }
}

// The prefetch role of a block: block b of n reads its share of the ranges in
// 16-byte pieces, consecutive lanes at consecutive addresses (a wave instruction
// covers 1 KB), every load of the thread issued before the first is used (offsets
// past a range read nothing: buffer loads); the loaded words only feed an empty
// asm statement, so the loads stay.
__device__ __forceinline__ void prefetch_lines(const Prefetch& pf, int b, int n) {
  const uint32_t step = (uint32_t)n * blockDim.x * 16u;
  const uint32_t base = ((uint32_t)b * blockDim.x + threadIdx.x) * 16u;
  u32x4 w[Prefetch::kMax][Prefetch::kPerThread];
#pragma unroll
  for (int r = 0; r < Prefetch::kMax; ++r) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(pf.ptr[r], pf.bytes[r]);
#pragma unroll
    for (int i = 0; i < Prefetch::kPerThread; ++i)
      w[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + i * step, 0, 0);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int r = 0; r < Prefetch::kMax; ++r)
#pragma unroll
    for (int i = 0; i < Prefetch::kPerThread; ++i) acc ^= w[r][i].x ^ w[r][i].y ^ w[r][i].z ^ w[r][i].w;
  asm volatile("" : : "v"(acc));
}

// Down projection and combine of token t and RB (64 or 32) output rows: wave
// i < k takes routed entry t k + i, wave k the shared expert, each over all
// K = I columns (256-column chunks, then the 128-column tail, in order); waves
// past the token's entries only join the barrier.  The block then adds the
// entries' gate-scaled rows in rank order, the shared expert's row and the
// residual.  32-row blocks double the blocks of a small batch.  sq_out (the
// next layer's norm): the squares' sums of the bf16 outputs per 16 rows,
// [token][H / 16].
template <int W, int NS, int TAIL, int RB>
__global__ __launch_bounds__(W * 64) void k_decode_down_combine_mx(MxFfnArgs a, const uint16_t* __restrict__ residual,
                                                                  float* __restrict__ out,
                                                                  uint16_t* __restrict__ out_bf16,
                                                                  float* __restrict__ sq_out, Prefetch pf) {
  constexpr int NV = 2 * NS + TAIL;   // activation chunks of K
  constexpr int S = RB / 16;          // 16-row MFMA groups of the block
  static_assert(RB == 64 || RB == 32, "64- or 32-row blocks");
  __shared__ __attribute__((aligned(16))) float red[W][S][64];
  const int nrg = a.H / RB;   // the launch's own rows of blocks; the ones after them prefetch
  if ((int)blockIdx.y >= nrg) {
    prefetch_lines(pf, (blockIdx.y - nrg) * gridDim.x + blockIdx.x, (gridDim.y - nrg) * gridDim.x);
    return;
  }
  const int tok = blockIdx.x, rg = blockIdx.y;
  // 64-row weight tile of the block, and the block's first row inside it
  const int tile = RB == 64 ? rg : rg >> 1, r0 = RB == 64 ? 0 : (rg & 1) * 32;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.I;
  const int Tk = a.T * a.k;
  const int n_ent = a.k + (a.with_shared ? 1 : 0);
  if (wv < n_ent) {
    const int r = wv < a.k ? tok * a.k + wv : Tk + tok;
    const MxALane AL = mx_a_lane(lane);
    const __amdgpu_buffer_rsrc_t rhd = buffer_rsrc(a.hdata + (size_t)r * mx_data_bytes(K), (uint32_t)mx_data_bytes(K));
    const __amdgpu_buffer_rsrc_t rhe = buffer_rsrc(a.hexps + (size_t)r * mx_exps_bytes(K), (uint32_t)mx_exps_bytes(K));
    MxAct X[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) X[v] = mx_load_act(rhd, rhe, AL, v);

    const int grp = r < Tk ? __builtin_amdgcn_readfirstlane(a.ids[r]) : a.E;
    const bool is_shared = grp == a.E;
    const MatRef& M = is_shared ? a.s2 : a.r2;
    const size_t eidx = is_shared ? 0 : (size_t)grp;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(M.codes + eidx * M.code_stride, (uint32_t)M.code_stride);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(M.scales + eidx * M.scale_stride, (uint32_t)(M.scale_stride * 2));
    const int n = lane & 15, q = lane >> 4;
    const int nch64 = K / 64, n128 = K / 128;

    u32x4 cw[NS + TAIL][S];
    uint32_t sc[NS + TAIL][S];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const uint32_t cso = (uint32_t)(((size_t)tile * nch64 + 4 * c) * 1024);
      const uint32_t sso = (uint32_t)(((size_t)tile * n128 + 2 * c) * 512);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        cw[c][s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(q * 1024 + (r0 + 16 * s + n) * 16), cso, 0);
        sc[c][s] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(((q >> 1) * 64 + r0 + 16 * s + n) * 8 + (q & 1) * 4), sso, 0);
      }
    }
    if (TAIL) {
      const int c = 2 * NS;
      const uint32_t cso = (uint32_t)(((size_t)tile * nch64 + 2 * c) * 1024);
      const uint32_t sso = (uint32_t)(((size_t)tile * n128 + c) * 512);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(
            rc, (uint32_t)((((q >> 1) * 64 + r0 + 16 * s + n) * 16) + 8 * (q & 1)), cso, 0);
        cw[NS][s] = u32x4{v[0], v[1], 0u, 0u};
        sc[NS][s] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)(((r0 + 16 * s + n) * 4 + q) * 2), sso, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
    const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    float y[S];
#pragma unroll
    for (int s = 0; s < S; ++s) y[s] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = v >> 1, pi = v & 1;   // the tail chunk (v = 2 NS) reads words 0, 1 of its own loads
      const mx_v8i A = mx_act_operand(X[v]);
      const mx_v4f off = mx_mfma(A, mx_minus_one(), (int)X[v].sa, zero);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const u32x4& w = cw[c][s];
        const mx_v4f o = mx_mfma(A, pi ? mx_weights(w.z, w.w) : mx_weights(w.x, w.y), (int)X[v].sa, off);
        y[s] = mx_accumulate(o, pi ? sc[c][s] >> 16 : sc[c][s] & 0xFFFFu, y[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) red[wv][s][(lane & 15) * 4 + (lane >> 4)] = y[s];
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < RB) {
    // row t: subgroup s = t / 16, row n = t % 16 of it; entries in rank order,
    // then the shared expert, then the residual
    const int s = t >> 4, nn = t & 15;
    float acc = 0.0f;
    for (int w = 0; w < n_ent; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[w][s][nn * 4]);
      const float e = ((v.x + v.y) + v.z) + v.w;
      acc += (w < a.k ? a.gates[(size_t)tok * a.k + w] : 1.0f) * e;
    }
    const size_t o = (size_t)tok * a.H + (size_t)rg * RB + t;
    if (residual) acc += bf16_to_f32(residual[o]);
    out[o] = acc;
    const uint32_t ob = f32_to_bf16_rne(acc);
    if (out_bf16) out_bf16[o] = (uint16_t)ob;
    if (sq_out) {
      // the block's rows are lanes 0 .. RB - 1 of wave 0; lane 16 j holds the
      // squares' sum of rows 16 j .. 16 j + 15
      const float sq = rms_row16_sums(bf16_to_f32(ob));
      if ((t & 15) == 0) sq_out[(size_t)tok * (a.H / 16) + rg * (RB / 16) + (t >> 4)] = sq;
    }
  }
}

bool decode_mx_ok(int H, int I, int q3) { return !q3 && H % 256 == 0 && I % 128 == 0 && H / 256 <= 20 && I <= 1024; }

// 32-row blocks when 64-row blocks would leave compute units idle (T = 1, 2).
hipError_t launch_decode_gateup_mx(const MxFfnArgs& a, hipStream_t s) {
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  const int ns = a.H / 256;
  const bool rows32 = entries * (a.I / 64) < 256;
  dim3 grid(entries, a.I / (rows32 ? 32 : 64));
#define MOE_GU_MX(SPW, VPL)                                                   \
  do {                                                                        \
    if (rows32)                                                               \
      MOE_LAUNCH((k_decode_gateup_mx<10, SPW, VPL, 32>), grid, dim3(640), 0, s, a); \
    else                                                                      \
      MOE_LAUNCH((k_decode_gateup_mx<10, SPW, VPL, 64>), grid, dim3(640), 0, s, a); \
  } while (0)
  if (ns <= 10) {
    if (a.E <= 512)
      MOE_GU_MX(1, 8);
    else
      MOE_GU_MX(1, 16);
  } else {
    if (a.E <= 512)
      MOE_GU_MX(2, 8);
    else
      MOE_GU_MX(2, 16);
  }
#undef MOE_GU_MX
  return hipGetLastError();
}

hipError_t launch_decode_down_combine_mx(const MxFfnArgs& a, const uint16_t* residual, float* out, uint16_t* out_bf16,
                                         float* sq_out, hipStream_t s, const Prefetch* pf) {
  const int n_ent = a.k + (a.with_shared ? 1 : 0);
  // 32-row blocks when 64-row ones would be very few (one token: 40 blocks at
  // H = 2560; measured 18.1 against 19.5 us a layer, while at four tokens 320
  // 32-row blocks were slower than 160 64-row ones)
  const bool rows32 = a.T * (a.H / 64) <= 64;
  const Prefetch p = pf ? *pf : Prefetch();
  // prefetch rows: about 160 blocks (on the compute units the launch's own blocks
  // leave free), enough for kPerThread 16-byte pieces per thread of the largest range
  const int waves = n_ent <= 11 ? 11 : 16;
  const uint32_t pieces = (p.max_bytes() + 15) / 16, per_row = (uint32_t)a.T * waves * 64 * Prefetch::kPerThread;
  const int prow = p.max_bytes() ? std::max((int)((pieces + per_row - 1) / per_row), (160 + a.T - 1) / a.T) : 0;
  dim3 grid(a.T, a.H / (rows32 ? 32 : 64) + prow);
  if (!decode_down_combine_mx_ok(a.I, a.k, a.with_shared)) return hipErrorInvalidValue;
#define MOE_DC_MX(W, NS, TL)                                                                                  \
  do {                                                                                                        \
    if (rows32)                                                                                               \
      MOE_LAUNCH((k_decode_down_combine_mx<W, NS, TL, 32>), grid, dim3(W * 64), 0, s, a, residual, out, out_bf16, \
                 sq_out, p);                                                                                  \
    else                                                                                                      \
      MOE_LAUNCH((k_decode_down_combine_mx<W, NS, TL, 64>), grid, dim3(W * 64), 0, s, a, residual, out, out_bf16, \
                 sq_out, p);                                                                                  \
  } while (0)
  const bool small = n_ent <= 11;
  switch (a.I) {
    case 512: if (small) MOE_DC_MX(11, 2, 0); else MOE_DC_MX(16, 2, 0); break;
    case 640: if (small) MOE_DC_MX(11, 2, 1); else MOE_DC_MX(16, 2, 1); break;
    case 768: if (small) MOE_DC_MX(11, 3, 0); else MOE_DC_MX(16, 3, 0); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_DC_MX
  return hipGetLastError();
}

bool decode_down_combine_mx_ok(int I, int k, int with_shared) {
  return (I == 512 || I == 640 || I == 768) && k + (with_shared ? 1 : 0) <= 16;
}

hipError_t launch_decode_down_mx(const MxFfnArgs& a, hipStream_t s) {
  const int entries = a.T * a.k + (a.with_shared ? a.T : 0);
  const int ns = a.I / 256, tail = (a.I % 256) ? 1 : 0;
  dim3 grid(entries, a.H / 64);
#define MOE_DOWN_MX(NS, TL) MOE_LAUNCH((k_decode_down_mx<NS, TL>), grid, dim3((NS + TL) * 64), 0, s, a)
  switch (ns * 2 + tail) {
    case 1: MOE_DOWN_MX(0, 1); break;
    case 2: MOE_DOWN_MX(1, 0); break;
    case 3: MOE_DOWN_MX(1, 1); break;
    case 4: MOE_DOWN_MX(2, 0); break;
    case 5: MOE_DOWN_MX(2, 1); break;
    case 6: MOE_DOWN_MX(3, 0); break;
    case 7: MOE_DOWN_MX(3, 1); break;
    case 8: MOE_DOWN_MX(4, 0); break;
    case 9: MOE_DOWN_MX(4, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_DOWN_MX
  return hipGetLastError();
}

}  // namespace moe

// Grouped-GEMM tiles of a few rows on the block-scaled fp8 x fp4 matrix cores.
//
// In a verify batch of many independent sequences (MTP drafts of 32 sequences,
// page "Strata Runs a 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU at up
// to 93 Tokens per Second", speculative-decoding paragraph) most selected experts
// are chosen by two or three tokens.  A 32-row fp16 tile dequantises its
// expert's whole weight matrix on the VALU (about twelve instructions per 512
// weights) whatever its rows; the decode form of mx.h turns 16 code bytes into
// fp4 operands with two instructions and pays one MFMA per row instead.  So a
// group of at most kMxTileRows rows gets one tile of this form: the same block
// shape, columns and outputs as the fp16 tile it replaces, the codes loaded once
// and every row's product run against them.
//
// Gate/up: wave w of column tile j owns h columns 128 j + 32 w + (0..31), i.e.
// 32 gate and 32 up weight rows (four 16-row MFMA groups), over all K = H in
// 256-column chunks (lane (n, q) loads the 16 code bytes of row n, 64-column
// chunk q and their two scales; two MFMAs per load: even blocks, odd blocks).
// Its epilogue writes h = SiLU(gate) up as the down tile's fp8-piece table.
// Down: wave w owns output rows 256 j + 64 w + (0..63) over K = I (256-column
// chunks and a 128-column tail) and writes fp32 rows, as the fp16 tile does.
// The rows' tables (x: per token, 256-column form; h: per sorted position, mixed
// form) are staged in LDS once per block.  Every float sum has a fixed order:
// chunks in K order, then the four lane groups of a row pairwise.
#pragma once

#include "device.h"
#include "internal.h"
#include "mfma.h"
#include "mx.h"

namespace moe {

// LDS bytes of the staged tables of kMxTileRows rows of K columns.
__host__ __device__ constexpr int mx_stage_bytes(int K) {
  return kMxTileRows * (int)(mx_data_bytes(K) + mx_exps_bytes(K));
}

// Copies the tables of `rows` rows into LDS, row j (source row src_j) at
// j * (data + exps bytes): its data part, then its scale bytes.  All of a
// thread's loads are issued before its first store.
template <int MAXK>
__device__ __forceinline__ void mx_stage(uint8_t* __restrict__ lds, const uint8_t* __restrict__ data,
                                         const uint8_t* __restrict__ exps, int K, int rows, const int (&src)[kMxTileRows]) {
  static_assert(kMxTileRows == 4, "the source row is picked from four");
  constexpr int IT = (mx_stage_bytes(MAXK) / 16 + 255) / 256;
  const int db = (int)mx_data_bytes(K), eb = (int)mx_exps_bytes(K);
  const int per = (db + eb) / 16;
  const int total = rows * per;
  u32x4 v[IT];
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int i = u * 256 + (int)threadIdx.x;
    if (i < total) {
      const int j = i / per, p = i - j * per;
      const int r = j == 0 ? src[0] : j == 1 ? src[1] : j == 2 ? src[2] : src[3];
      const uint8_t* s = 16 * p < db ? data + (size_t)r * db + 16 * p : exps + (size_t)r * eb + (16 * p - db);
      v[u] = *reinterpret_cast<const u32x4*>(s);
    }
  }
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int i = u * 256 + (int)threadIdx.x;
    if (i < total) {
      const int j = i / per, p = i - j * per;
      *reinterpret_cast<u32x4*>(lds + j * (db + eb) + 16 * p) = v[u];
    }
  }
}

// Activation operand of staged row j, table chunk v, for this lane: the lane
// holds one 16-byte half (or none) of the operand, so one LDS read and a mask
// per half give the block-diagonal operand that mx_load_act reads from memory.
struct MxLdsLane {
  uint32_t off;        // byte offset of the lane's 16 bytes within a chunk
  uint32_t mlo, mhi;   // all ones if the lane holds operand dwords 0..3 / 4..7
  uint32_t exp;        // scale byte of row m = lane % 16
};

__device__ __forceinline__ MxLdsLane mx_lds_lane(int lane) {
  const MxALane AL = mx_a_lane(lane);
  const bool lo = AL.off_lo < 0x80000000u, hi = AL.off_hi < 0x80000000u;
  MxLdsLane L;
  L.off = lo ? AL.off_lo : (hi ? AL.off_hi : 0u);
  L.mlo = lo ? ~0u : 0u;
  L.mhi = hi ? ~0u : 0u;
  L.exp = AL.exp_off;
  return L;
}

__device__ __forceinline__ mx_v8i mx_lds_act(const uint8_t* __restrict__ row, int db, int v, const MxLdsLane& L,
                                             int& sa) {
  const u32x4 d = *reinterpret_cast<const u32x4*>(row + v * 128 * kMxPieces + L.off);
  sa = row[db + v * 16 + L.exp];
  mx_v8i a;
  a[0] = (int)(d.x & L.mlo);
  a[1] = (int)(d.y & L.mlo);
  a[2] = (int)(d.z & L.mlo);
  a[3] = (int)(d.w & L.mlo);
  a[4] = (int)(d.x & L.mhi);
  a[5] = (int)(d.y & L.mhi);
  a[6] = (int)(d.z & L.mhi);
  a[7] = (int)(d.w & L.mhi);
  return a;
}

// Sum over the four lane groups of a row (lanes n, n + 16, n + 32, n + 48):
// the same bits in all four lanes.
__device__ __forceinline__ float mx_row_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Codes and scales of a wave's four 16-row groups for one 256-column chunk.
struct MxChunk {
  u32x4 c[4];
  uint32_t s[4];
};

// Gate/up of one tile for this wave's h columns c0 .. c0 + 31 (c0 % 32 == 0):
// gate rows c0 + (0..31) and up rows I + c0 + (0..31) of the expert's W13
// (codes rc, scales rs), K = H % 256 == 0, D chunks of codes in flight.  stage():
// the block's staging of the rows' x tables into lds (with its barrier), called
// once the first chunks' loads are issued; h rows m0 + j of hdata / hexps (I
// columns, mixed form).
template <int D, typename Stage>
__device__ __forceinline__ void mx_tile_gateup(const uint8_t* __restrict__ lds, int rows, int H, int I, int c0,
                                               __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int m0,
                                               uint8_t* __restrict__ hdata, uint8_t* __restrict__ hexps,
                                               Stage&& stage) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int db = (int)mx_data_bytes(H), rb = db + (int)mx_exps_bytes(H);
  const int ns = H / 256, nch64 = H / 64, n128 = H / 128;
  const int ngate = c0 >> 6, nup = (I + c0) >> 6, ro = c0 & 63;
  uint32_t vc[2], vs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = ro + 16 * h + n;
    vc[h] = (uint32_t)(q * 1024 + row * 16);
    vs[h] = (uint32_t)(((q >> 1) * 64 + row) * 8 + (q & 1) * 4);
  }
  // groups 0, 1: gate rows (ro, ro + 16); 2, 3: up rows.  Loads past the last
  // chunk re-load it (every load unconditional: exact wait counts).
  auto load = [&](int c, MxChunk& B) {
    c = c < ns ? c : ns - 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ng = g < 2 ? ngate : nup;
      B.c[g] = __builtin_amdgcn_raw_buffer_load_b128(rc, vc[g & 1], (ng * nch64 + 4 * c) * 1024, 0);
      B.s[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs[g & 1], (ng * n128 + 2 * c) * 512, 0);
    }
  };
  const MxLdsLane L = mx_lds_lane(lane);
  const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float y[kMxTileRows][4];
#pragma unroll
  for (int j = 0; j < kMxTileRows; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) y[j][g] = 0.0f;

  // chunk c from B: its fp4 operands and scales are taken out of B, B is
  // refilled with chunk c + D, then every row's products
  auto chunk = [&](MxChunk& B, int c) {
    mx_v8i W[2][4];
    float sc[2][4];   // the fp16 block scales of this lane's (row, even / odd block)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      W[0][g] = mx_weights(B.c[g].x, B.c[g].y);
      W[1][g] = mx_weights(B.c[g].z, B.c[g].w);
      sc[0][g] = fp16_to_f32(B.s[g] & 0xFFFFu);
      sc[1][g] = fp16_to_f32(B.s[g] >> 16);
    }
    load(c + D, B);
#pragma unroll
    for (int j = 0; j < kMxTileRows; ++j) {
      if (j < rows) {
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
          int sa;
          const mx_v8i A = mx_lds_act(lds + j * rb, db, 2 * c + pi, L, sa);
          const mx_v4f off = mx_mfma(A, mx_minus_one(), sa, zero);   // -2 sum v per (piece, block)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const mx_v4f o = mx_mfma(A, W[pi][g], sa, off);
            y[j][g] = fmaf(sc[pi][g], (o[0] + o[1]) + (o[2] + o[3]), y[j][g]);
          }
        }
      }
    }
  };
  MxChunk B[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, B[d]);
  stage();
  int c = 0;
  for (; c + D <= ns; c += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) chunk(B[d], c + d);
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (c + d < ns) chunk(B[d], c + d);

  // rows summed over the lane groups; lane L < 32 holds h column c0 + L (lanes
  // 32..63 the same values: they take part in the block maximum, store nothing)
  const int l32 = lane & 31;
#pragma unroll
  for (int j = 0; j < kMxTileRows; ++j) {
    if (j < rows) {
      float r[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) r[g] = mx_row_sum(y[j][g]);
      const float gv = l32 < 16 ? r[0] : r[1], uv = l32 < 16 ? r[2] : r[3];
      const float hv = gv / (1.0f + expf(-gv)) * uv;
      mx_emit(hv, m0 + j, mx_slot_mixed(c0 >> 5, I), mx_pos_of_weight(l32), I, hdata, hexps, lane < 32);
    }
  }
}

// Down projection of one tile for this wave's output rows o0 .. o0 + 63
// (o0 % 64 == 0) of the expert's W2, K = I = 256 NS + 128 TAIL; every code load
// is issued before stage() puts the rows' h tables into lds; fp32 rows m0 + j of
// y (H columns).
template <int NS, int TAIL, typename Stage>
__device__ __forceinline__ void mx_tile_down(const uint8_t* __restrict__ lds, int rows, int H, int o0,
                                             __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int m0,
                                             float* __restrict__ y_out, Stage&& stage) {
  constexpr int K = 256 * NS + 128 * TAIL;
  constexpr int NV = 2 * NS + TAIL;   // table chunks of K
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int db = (int)mx_data_bytes(K), rb = db + (int)mx_exps_bytes(K);
  constexpr int nch64 = K / 64, n128 = K / 128;
  const int ng = o0 >> 6;
  u32x4 cw[NS + TAIL][4];
  uint32_t sc[NS + TAIL][4];
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = 16 * g + n;
      cw[c][g] = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(q * 1024 + row * 16), (ng * nch64 + 4 * c) * 1024, 0);
      sc[c][g] = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(((q >> 1) * 64 + row) * 8 + (q & 1) * 4),
                                                      (ng * n128 + 2 * c) * 512, 0);
    }
  if (TAIL) {
    // 128-column tail: lane (n, q) reads block q of row n (8 bytes) and its scale
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = 16 * g + n;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(
          rc, (uint32_t)((((q >> 1) * 64 + row) * 16) + 8 * (q & 1)), (ng * nch64 + 4 * NS) * 1024, 0);
      cw[NS][g] = u32x4{v[0], v[1], 0u, 0u};
      sc[NS][g] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)((row * 4 + q) * 2), (ng * n128 + 2 * NS) * 512, 0);
    }
  }
  stage();
  const MxLdsLane L = mx_lds_lane(lane);
  const mx_v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float y[kMxTileRows][4];
#pragma unroll
  for (int j = 0; j < kMxTileRows; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) y[j][g] = 0.0f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = v >> 1, pi = v & 1;   // the tail chunk (v = 2 NS) reads words 0, 1 of its own loads
    mx_v8i W[4];
    float s[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      W[g] = pi ? mx_weights(cw[c][g].z, cw[c][g].w) : mx_weights(cw[c][g].x, cw[c][g].y);
      s[g] = fp16_to_f32(pi ? sc[c][g] >> 16 : sc[c][g] & 0xFFFFu);
    }
#pragma unroll
    for (int j = 0; j < kMxTileRows; ++j) {
      if (j < rows) {
        int sa;
        const mx_v8i A = mx_lds_act(lds + j * rb, db, v, L, sa);
        const mx_v4f off = mx_mfma(A, mx_minus_one(), sa, zero);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const mx_v4f o = mx_mfma(A, W[g], sa, off);
          y[j][g] = fmaf(s[g], (o[0] + o[1]) + (o[2] + o[3]), y[j][g]);
        }
      }
    }
  }
  // lane l = 16 q + n stores output row o0 + l: group q, row n
#pragma unroll
  for (int j = 0; j < kMxTileRows; ++j) {
    if (j < rows) {
      float r[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) r[g] = mx_row_sum(y[j][g]);
      const float val = q == 0 ? r[0] : q == 1 ? r[1] : q == 2 ? r[2] : r[3];
      y_out[(size_t)(m0 + j) * H + o0 + lane] = val;
    }
  }
}

}  // namespace moe

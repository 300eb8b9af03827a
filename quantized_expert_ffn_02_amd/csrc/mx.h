// Block-scaled fp8 x fp4 matrix-core form of the 2-bit dequant GEMV
// (v_mfma_scale_f32_16x16x128_f8f6f4, gfx950).
//
// Weights.  A 2-bit code c (weight c - 2) placed in the low two bits of an fp4
// (e2m1) nibble reads as c / 2 exactly (0, 0.5, 1, 1.5), so a u32 word of 16
// codes (weight j at bits 2j..2j+1) becomes two fp4 words with one AND and one
// shift-AND: w & 0x33333333 holds the even weights (nibble i = weight 2i),
// (w >> 2) & 0x33333333 the odd ones.  A 32-weight block (two words) is one
// lane's operand: position p of the block holds weight
//   wt(p) = 16 (p / 16) + (p % 16 < 8 ? 2 (p % 8) : 2 (p % 8) + 1).
//
// Activations.  A value v of a 32-column block is a sum of four e4m3 pieces,
// fixed point against the block: with e the exponent that maps the block's
// largest magnitude into [128, 256), piece j is the remainder rounded (to
// nearest even) to a multiple of 16 * 2^(e - 5j), stored as k_j * 16 with
// |k_j| <= 16 and exponent e_j = e - 5j.  The remainder after four pieces is at
// most 2^-19 of the block's largest value.  Every nonzero term that one MFMA
// output adds is then k * 8 * 2^e_j with |k| <= 48 (codes / 2 are 0.5 .. 1.5):
// a narrow range in which the matrix core's accumulation is exact (across a
// wide range of magnitudes it is not: about 13 bits were measured).  The MFMA's
// per-row E8M0 scale carries 2^(e_j + 1): the + 1 turns c / 2 back into c.
//
// MFMA rows.  In the 16 x 16 x 128 form, row m = 4 b + j of the activation
// operand holds piece j of block b of a 128-column chunk (zero outside block
// b), and the 16 columns are 16 weight rows.  Output lane l then holds weight
// row l % 16 and block b = l / 16, pieces j = 0..3 in its four registers:
//   sum_j out_j = sum_k c_k v_k  over the block,
// The code offset comes from the accumulator input: one MFMA per chunk against
// an fp4 operand of -1.0 everywhere gives -2 sum_k v_k for every (row, block),
// and each weight MFMA starts from it, so its outputs sum to
//   sum_j out_j = sum_k (c_k - 2) v_k  over the block,
// and the block's contribution to the GEMV is s * sum_j out_j with s the
// block's fp16 weight scale: three adds and one fused multiply-add per (weight
// row, block), against one bf16 pair operation per two weights in the VALU form
// (device.h).
//
// Operand lane layouts (measured on gfx950): the fp4 operand's lane l holds
// row / column l % 16 and K positions 32 (l / 16) + n at nibble n (low nibble
// first); the fp8 operand's lane l holds row / column l % 16 with byte J at
// K = 64 (J / 16) + 16 (l / 16) + J % 16; the scale of lane l applies to row /
// column l % 16 and K block l / 16 (32 positions) of its operand.  So piece j
// of block b, half h (positions 16 h .. 16 h + 15) sits in lane
// 16 (2 (b % 2) + h) + 4 b + j, bytes 16 (b / 2) .. 16 (b / 2) + 15.
//
// Table of a row of K columns (K % 128 == 0), per chunk c of four blocks (the
// blocks of a 128-column chunk, or the even or odd blocks of 256 columns):
//   data [chunk][block 4][half 2][piece 4][16 bytes]  e4m3 pieces, position
//        order of the fp4 operand (byte i of half h = position 16 h + i)
//   exps [chunk][16 bytes]  E8M0 scale byte of row m = 4 b + j (127 + e_j + 1)
#pragma once

#include "device.h"

namespace moe {

typedef int mx_v8i __attribute__((ext_vector_type(8)));
typedef float mx_v4f __attribute__((ext_vector_type(4)));

static constexpr int kMxPieces = 4;

// Bytes of a row's table parts for K columns.
__host__ __device__ constexpr size_t mx_data_bytes(int K) { return (size_t)(K / 128) * 128 * kMxPieces; }
__host__ __device__ constexpr size_t mx_exps_bytes(int K) { return (size_t)(K / 128) * 16; }

// Block position of weight index w (0..31) in the fp4 operand order.
__device__ __forceinline__ int mx_pos_of_weight(int w) {
  const int r = w & 15;
  return (w & 16) | ((r & 1) ? 8 + (r >> 1) : (r >> 1));
}
// Weight index at block position p.
__device__ __forceinline__ int mx_weight_at(int p) {
  const int i = p & 15;
  return (p & 16) | (i < 8 ? 2 * i : 2 * (i - 8) + 1);
}

// Largest |v| over each 32-lane half of the wave, in every lane of that half:
// DPP steps inside each 16-lane row (magnitudes as unsigned words order like
// the floats; moves from outside the row read 0), then the four row results.
__device__ __forceinline__ float half_wave_max_abs(float v) {
  uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));    // quad_perm 1,0,3,2
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));    // quad_perm 2,3,0,1
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, true));   // row_ror 4
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, true));   // row_ror 8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)u, 48);
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? max(r0, r1) : max(r2, r3));
}

// Pieces of the value v held by this lane; the 32 lanes of each half wave form
// one block (all 64 lanes must call).  p[j]: e4m3 bytes; sb[j]: E8M0 scale
// bytes (127 + e_j + 1).  Piece j is k_j * 16 * 2^e_j with k_j = rint(r / u_j),
// u_j = 2^(e_j + 4) its unit (u_j and 1 / u_j normal floats for every e here, so
// both products are exact), r = fma(-k_j, u_j, r) the exact remainder; 16 k_j
// (|k_j| <= 16) is an e4m3 value exactly, converted two at a time by the
// hardware (no rounding happens).
__device__ __forceinline__ void mx_pieces(float v, uint32_t (&p)[kMxPieces], uint32_t (&sb)[kMxPieces]) {
  const float m = half_wave_max_abs(v);
  int e = (int)((__float_as_uint(m) >> 23) & 255u) - 134;   // floor(log2 m) - 7
  e = m > 0.0f ? (e < -113 ? -113 : e) : 0;                  // e - 15 stays a valid scale
  float u = __uint_as_float((uint32_t)(e + 4 + 127) << 23);         // 2^(e_0 + 4)
  float ui = __uint_as_float((uint32_t)(127 - (e + 4)) << 23);      // 2^-(e_0 + 4)
  float r = v, k16[kMxPieces];
#pragma unroll
  for (int j = 0; j < kMxPieces; ++j) {
    const float k = __builtin_rintf(r * ui);
    r = fmaf(-k, u, r);
    k16[j] = 16.0f * k;
    sb[j] = (uint32_t)(128 + e - 5 * j);
    u *= 0.03125f;
    ui *= 32.0f;
  }
  static_assert(kMxPieces == 4, "two packed conversions");
  const uint32_t b01 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(k16[0], k16[1], 0, false);
  const uint32_t b23 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(k16[2], k16[3], 0, false);
  p[0] = b01 & 0xFFu;
  p[1] = (b01 >> 8) & 0xFFu;
  p[2] = b23 & 0xFFu;
  p[3] = (b23 >> 8) & 0xFFu;
}

// fp4 operand of a 32-weight block from its two code words.
__device__ __forceinline__ mx_v8i mx_weights(uint32_t w0, uint32_t w1) {
  mx_v8i b;
  b[0] = (int)(w0 & 0x33333333u);
  b[1] = (int)((w0 >> 2) & 0x33333333u);
  b[2] = (int)(w1 & 0x33333333u);
  b[3] = (int)((w1 >> 2) & 0x33333333u);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// fp4 operand of -1.0 at every position (the code offset).
__device__ __forceinline__ mx_v8i mx_minus_one() {
  mx_v8i b;
  b[0] = b[1] = b[2] = b[3] = (int)0xAAAAAAAAu;
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// One 16 x 16 x 128 product: activation pieces (fp8, per-row scales sa) times
// 16 weight rows (fp4, unit scales), plus c.
__device__ __forceinline__ mx_v4f mx_mfma(const mx_v8i& a, const mx_v8i& b, int sa, const mx_v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
}

// y + s * (sum of the four pieces' outputs) for this lane's (weight row, block);
// s is the block's fp16 weight scale.
__device__ __forceinline__ float mx_accumulate(const mx_v4f& o, uint32_t scale16, float y) {
  return fmaf(fp16_to_f32(scale16), (o[0] + o[1]) + (o[2] + o[3]), y);
}

// Per-lane constants for reading a row's activation operand of one chunk
// (chunk base in the scalar offset): the byte offsets of this lane's 16 bytes
// in the data part, or an offset past the end (the buffer load then returns
// zero) for the halves it does not hold.
struct MxALane {
  uint32_t off_lo, off_hi;   // data offsets for operand dwords 0..3 and 4..7
  uint32_t exp_off;          // byte of the scale of row m = lane % 16
};

__device__ __forceinline__ MxALane mx_a_lane(int lane) {
  const int m = lane & 15, b = m >> 2, j = m & 3, g = lane >> 4;
  const bool act = (g >> 1) == (b & 1);
  const uint32_t off = (uint32_t)((((b * 2 + (g & 1)) * kMxPieces + j) * 16));
  MxALane L;
  L.off_lo = act && (b >> 1) == 0 ? off : 0x80000000u;
  L.off_hi = act && (b >> 1) == 1 ? off : 0x80000000u;
  L.exp_off = (uint32_t)m;
  return L;
}

// Table slot of 32-column block B: the 128-column chunk form puts block B in
// slot B (chunk B / 4, block B % 4 of it).  The 256-column form (two MFMAs per
// 16-byte code load: even blocks, then odd blocks of the 256 columns) puts
// block B in chunk 2 (B / 8) + B % 2, block (B % 8) / 2 of it.
__host__ __device__ constexpr int mx_slot128(int B) { return B; }
__host__ __device__ constexpr int mx_slot256(int B) { return 4 * (2 * (B >> 3) + (B & 1)) + ((B & 7) >> 1); }
// Mixed form for K = 256 ns + 128 t: the 256-column form for the first 256 ns
// columns, a 128-column chunk for the rest.
__host__ __device__ constexpr int mx_slot_mixed(int B, int K) { return B < (K / 256) * 8 ? mx_slot256(B) : B; }

// Activation table of this lane's value v (this half wave holds the block in
// table slot `slot`, this lane position p of the block) in row `row`: pieces
// and scale bytes.  Every lane takes part in the block maximum; only lanes
// with `store` write.
__device__ __forceinline__ void mx_emit(float v, int row, int slot, int p, int K, uint8_t* __restrict__ data,
                                        uint8_t* __restrict__ exps, bool store = true) {
  uint32_t pc[kMxPieces], sb[kMxPieces];
  mx_pieces(v, pc, sb);
  if (!store) return;
  uint8_t* __restrict__ d =
      data + (size_t)row * mx_data_bytes(K) + (size_t)((slot * 2 + (p >> 4)) * kMxPieces) * 16 + (p & 15);
#pragma unroll
  for (int j = 0; j < kMxPieces; ++j) d[j * 16] = (uint8_t)pc[j];
  if (p == 0)
    reinterpret_cast<uint32_t*>(exps + (size_t)row * mx_exps_bytes(K))[slot] =
        sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
}

// Table of T rows of bf16 x (256-column form) built by blocks blk of nblk
// (256 threads each): element it = (row, column) in the table's column order
// (the thread of block position p reads the weight index at p).  A pass gives
// each thread kMxTablePer elements, 256 apart, whose loads are all issued
// before the first piece is made.  T H is a multiple of 64, so the waves are
// whole and all 64 lanes of each take part in the block maxima.
static constexpr int kMxTablePer = 4;

__host__ __device__ constexpr int mx_table_blocks(int T, int H, int cap) {
  return (T * H + 256 * kMxTablePer - 1) / (256 * kMxTablePer) < cap ? (T * H + 256 * kMxTablePer - 1) / (256 * kMxTablePer)
                                                                    : cap;
}

__device__ __forceinline__ void mx_table_pass(const uint16_t* __restrict__ x, int T, int H, uint8_t* __restrict__ data,
                                              uint8_t* __restrict__ exps, int blk, int nblk) {
  const int items = T * H;
  for (int base = blk * 256 * kMxTablePer; base < items; base += nblk * 256 * kMxTablePer) {
    float v[kMxTablePer];
#pragma unroll
    for (int u = 0; u < kMxTablePer; ++u) {
      const int it = base + u * 256 + (int)threadIdx.x;
      v[u] = 0.0f;
      if (it < items) {
        const int row = it / H, col = it - row * H;
        v[u] = bf16_to_f32(x[(size_t)row * H + (col & ~31) + mx_weight_at(col & 31)]);
      }
    }
#pragma unroll
    for (int u = 0; u < kMxTablePer; ++u) {
      const int it = base + u * 256 + (int)threadIdx.x;
      if (it < items) {
        const int row = it / H, col = it - row * H;
        mx_emit(v[u], row, mx_slot256(col >> 5), col & 31, H, data, exps);
      }
    }
  }
}

}  // namespace moe

// Device helpers for the gfx950 kernels: bf16/fp16 conversions, the packed
// bf16 dot product, wave64 reductions, and the 2-bit block dot product used by
// every dequant-GEMV kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN keeps a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : r;   // NaN stays a quiet NaN
}

__device__ __forceinline__ float fp16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// acc + a.lo*b.lo + a.hi*b.hi over packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(moe_bf16x2, a),
                                         __builtin_bit_cast(moe_bf16x2, b), acc, false);
}

// A constant held in a VGPR, so that (x & m) | magic can be one v_and_or_b32
// (gfx9 VOP3 encodings take no literal operand).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// Raw buffer resource (gfx9 layout, stride 0) over `bytes` bytes from `base`:
// loads take a 32-bit per-lane offset and a wave-uniform scalar offset, and
// return zero past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}

// Sum over the 64 lanes in a fixed order (wave-uniform result): DPP adds
// inside each 16-lane row (quad exchanges, then rotations by 4 and 8), then
// the four row sums in row order.
__device__ __forceinline__ float wave_sum_rows(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));    // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));    // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));   // row_ror 4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));   // row_ror 8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// RMSNorm of a bf16 row, one definition for every kernel that computes it:
// the squares of a 64-column group (lane = column, rounded squares, no
// contraction into the adds) summed by wave_sum_rows; the group sums
// (lane = group, G = H / 64 <= 64) summed the same way; then
// 1 / sqrt(sum / H + eps).  The fused stack path gets the same bits as the
// standalone norm.
__device__ __forceinline__ float rms_group_sum(float v) {
#pragma clang fp contract(off)
  const float sq = v * v;
  return wave_sum_rows(sq);
}
__device__ __forceinline__ float rms_inv_from_groups(float group_sum_or_zero, int H, float eps) {
#pragma clang fp contract(off)
  return 1.0f / sqrtf(wave_sum_rows(group_sum_or_zero) / (float)H + eps);
}

// The squares' sums of the 16-column rows of a 64-column group, as
// rms_group_sum forms them (each at lane 16 j of the 16-lane row j; a kernel with
// 32 columns in lanes 0..31 gets rows 0 and 1 with the same bits).
__device__ __forceinline__ float rms_row16_sums(float v) {
#pragma clang fp contract(off)
  float q = v * v;
  q += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(q), 0xB1, 0xF, 0xF, true));
  q += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(q), 0x4E, 0xF, 0xF, true));
  q += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(q), 0x124, 0xF, 0xF, true));
  q += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(q), 0x128, 0xF, 0xF, true));
  return q;
}

// RMSNorm scale of row t from its 16-column sums sq[t * (H / 16) + j]: group g
// adds its four in the order rms_group_sum does, then the groups as
// rms_inv_from_groups does.  Wave-uniform, every lane must call.
__device__ __forceinline__ float row_inv_rms(const float* __restrict__ sq, int t, int H, float eps) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, G = H / 64;
  float g = 0.0f;
  if (lane < G) {
    const float4 r = *reinterpret_cast<const float4*>(sq + (size_t)t * (H / 16) + 4 * lane);
    g = ((r.x + r.y) + r.z) + r.w;
  }
  return rms_inv_from_groups(g, H, eps);
}

// Row exponent of the grouped GEMMs' fp16 activation copy: a = -floor(log2 m)
// for the largest magnitude m of a bf16 row, given as the largest low 15 bits of
// its bit patterns (|x| orders as those bits for finite bf16); the row is
// stored as x 2^a, its largest magnitude in [1, 2).  Zero, inf or NaN maxima
// give 0.
__device__ __forceinline__ int bf16_row_exponent(uint32_t maxbits15) {
  if (maxbits15 == 0u || maxbits15 >= 0x7F80u) return 0;
  const int be = (int)(maxbits15 >> 7);
  const int e2 = be ? be - 127 : (31 - __builtin_clz(maxbits15 & 0x7Fu)) - 133;   // floor(log2 m)
  return -e2;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, MOE_WAVE));
  return m;
}

typedef __bf16 moe_bf16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 values (one u32) times s, rounded to bf16 (nearest even).
__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, float s) {
  const moe_bf16x2_t r = {(__bf16)(bf16_to_f32(w & 0xFFFFu) * s), (__bf16)(bf16_to_f32(w >> 16) * s)};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}

// ---------------------------------------------------------------------------
// 2-bit block dot product ("magic pair" form).
//
// A 32-weight block is two u32 words of 16 codes each (weight j of a word at
// bits 2j..2j+1).  For pair index j in 0..7 the word holds weight j in its low
// half and weight j + 8 in its high half.  Three code positions of each half
// (bits 0-1, 2-3, 4-5) lie inside a bf16 significand; OR-ing the exponent of
// 128.0 onto them gives the bf16 pair (128 + c_j * 2^p, 128 + c_{j+8} * 2^p)
// with no conversion instruction.  The activation pair table holds
// (x_j * 2^-p, x_{j+8} * 2^-p) (exact: scaling by a power of two), so one
// dot2 yields x*c plus the constant 128 * 2^-p * x, and the per-block init
// value  -(sum_k (128 * 2^-p(k) + 2) * x_k)  removes both that constant and
// the code offset 2.  Result: sum_k x_k * (c_k - 2) over the block.
//
//   pair j : 0 1 2 | 3 4 5 | 6 7
//   shift  : 0 0 0 | 6 6 6 | 12 12
//   p      : 0 2 4 | 0 2 4 | 0 2
// ---------------------------------------------------------------------------
struct Q2Masks {
  uint32_t m0, m1, m2, magic;
};

__device__ __forceinline__ Q2Masks q2_masks() {
  Q2Masks m;
  m.m0 = vgpr_const(0x00030003u);
  m.m1 = vgpr_const(0x000C000Cu);
  m.m2 = vgpr_const(0x00300030u);
  m.magic = vgpr_const(0x43004300u);
  return m;
}

// acc + sum over the 16 weights of word w of x * c (plus the magic constant
// term), with xp the 8 activation pairs of this word.
__device__ __forceinline__ float q2_word_dot(uint32_t w, const uint32_t* __restrict__ xp, float acc,
                                             const Q2Masks& M) {
  const uint32_t a = w, b = w >> 6, c = w >> 12;
  acc = dot2_bf16((a & M.m0) | M.magic, xp[0], acc);
  acc = dot2_bf16((a & M.m1) | M.magic, xp[1], acc);
  acc = dot2_bf16((a & M.m2) | M.magic, xp[2], acc);
  acc = dot2_bf16((b & M.m0) | M.magic, xp[3], acc);
  acc = dot2_bf16((b & M.m1) | M.magic, xp[4], acc);
  acc = dot2_bf16((b & M.m2) | M.magic, xp[5], acc);
  acc = dot2_bf16((c & M.m0) | M.magic, xp[6], acc);
  acc = dot2_bf16((c & M.m1) | M.magic, xp[7], acc);
  return acc;
}

// ---------------------------------------------------------------------------
// 3-bit block dot product.  Codes c = lo + 4 hi; lo uses the 2-bit form above,
// hi is a bit plane whose 32-bit word d covers lo-words 2d and 2d+1:
// bits j / 16 + j (j < 8) hold the hi bits of weights j / j + 8 of word 2d, and
// bits 8 + j / 24 + j those of word 2d + 1.  For word 2d the pair of bit
// position j (j = 0..6) is used in place (it lies inside a bf16 significand:
// magic 128, value 128 + hi * 2^j); position 7 is shifted down to 0.  Word
// 2d + 1 first shifts h right by 8.  The hi pair table holds
// (4 x_j 2^-q, 4 x_{j+8} 2^-q) with q = j (j < 7) and q = 0 (j = 7), so each dot
// adds 4 * x * hi plus the constant 512 * 2^-q * x, which the init removes.
// ---------------------------------------------------------------------------
struct Q3Masks {
  uint32_t bit[7];
  uint32_t magic;
};

__device__ __forceinline__ Q3Masks q3_masks() {
  Q3Masks m;
#pragma unroll
  for (int j = 0; j < 7; ++j) m.bit[j] = vgpr_const(0x00010001u << j);
  m.magic = vgpr_const(0x43004300u);
  return m;
}

__device__ __forceinline__ float q3_hi_dot(uint32_t h, const uint32_t* __restrict__ xp, float acc,
                                           const Q3Masks& M) {
#pragma unroll
  for (int j = 0; j < 7; ++j) acc = dot2_bf16((h & M.bit[j]) | M.magic, xp[j], acc);
  acc = dot2_bf16(((h >> 7) & M.bit[0]) | M.magic, xp[7], acc);
  return acc;
}

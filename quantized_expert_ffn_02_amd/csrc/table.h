// Activation pair tables for the dequant-GEMV kernels (see device.h for the
// "magic pair" arithmetic they serve).  For every input row and 32-column
// block the table holds SETS x 16 packed bf16 pairs and one fp32 init value:
// sets are [split][plane] with split = (hi, lo) parts of an fp32 input (one
// part for bf16 input) and plane = (2-bit codes, 3-bit high bits).
#pragma once

#include "device.h"

namespace moe {

// exponent shift p of lo-plane pair j and q of hi-plane pair j (device.h tables)
__device__ __forceinline__ int lo_shift(int j) {
  // {0, 2, 4, 0, 2, 4, 0, 2} packed 3 bits per entry (no memory table)
  return (0x422110 >> (3 * j)) & 7;
}
__device__ __forceinline__ int hi_shift(int j) { return j < 7 ? j : 0; }

// ---------------------------------------------------------------------------
// Activation tables.  One block of 256 threads per input row; 16 threads per
// 32-column block: thread (wi, j) handles the pair (16 wi + j, 16 wi + j + 8).
// Sets per block: [split][plane] with split = hi, lo (fp32 input only) and
// plane = lo codes, hi bits (Q3 only).
// ---------------------------------------------------------------------------
template <bool Q3, bool SPLIT>
__device__ void prep_row(const float v0, const float v1, int row, int b, int wi, int j, int nblk,
                         uint32_t* __restrict__ pairs, float* __restrict__ init) {
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * (SPLIT ? 2 : 1);
  const float sp = ldexpf(1.0f, -lo_shift(j));
  const float sq = ldexpf(4.0f, -hi_shift(j));
  float hi0 = v0, hi1 = v1, lo0 = 0.0f, lo1 = 0.0f;
  if (SPLIT) {
    hi0 = bf16_to_f32(f32_to_bf16_rne(v0));
    hi1 = bf16_to_f32(f32_to_bf16_rne(v1));
    lo0 = bf16_to_f32(f32_to_bf16_rne(v0 - hi0));
    lo1 = bf16_to_f32(f32_to_bf16_rne(v1 - hi1));
  }
  uint32_t* __restrict__ dst = pairs + ((size_t)row * nblk + b) * (SETS * 16) + wi * 8 + j;
  const float parts0[2] = {hi0, lo0}, parts1[2] = {hi1, lo1};
#pragma unroll
  for (int s = 0; s < (SPLIT ? 2 : 1); ++s) {
    dst[(s * PLANES) * 16] = f32_to_bf16_rne(parts0[s] * sp) | (f32_to_bf16_rne(parts1[s] * sp) << 16);
    if (Q3)
      dst[(s * PLANES + 1) * 16] = f32_to_bf16_rne(parts0[s] * sq) | (f32_to_bf16_rne(parts1[s] * sq) << 16);
  }
  // init = -sum_k (128 2^-p + [512 2^-q] + offset) * value_k over the block's 32 weights
  const float mult = 128.0f * sp + (Q3 ? 128.0f * sq + 4.0f : 2.0f);
  float term = mult * (hi0 + lo0) + mult * (hi1 + lo1);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) term += __shfl_xor(term, off, 16);
  if (wi == 0 && j == 0) init[(size_t)row * nblk + b] = -term;
}


// Table entry (b, wi, j) of a bf16 row x[row, 0..K).
__device__ __forceinline__ void prep_x_item(const uint16_t* __restrict__ x, int row, int K, int b, int wi, int j,
                                            bool q3, uint32_t* __restrict__ pairs, float* __restrict__ init) {
  const int k0 = b * 32 + wi * 16 + j;
  const float v0 = bf16_to_f32(x[(size_t)row * K + k0]);
  const float v1 = bf16_to_f32(x[(size_t)row * K + k0 + 8]);
  if (q3)
    prep_row<true, false>(v0, v1, row, b, wi, j, K / 32, pairs, init);
  else
    prep_row<false, false>(v0, v1, row, b, wi, j, K / 32, pairs, init);
}

// Down-projection table entries written straight from the gate/up epilogue: a
// full wave holds h for 64 consecutive columns (two 32-column blocks) of row
// ``row``; lane L owns column 64 * rg + L.  Same arithmetic as prep_row with the
// hi/lo split; the init sums run over the 32 lanes of each block.
template <bool Q3>
__device__ __forceinline__ void emit_down_table(float h, int row, int rg, int K, uint32_t* __restrict__ pairs,
                                                float* __restrict__ init) {
  constexpr int PLANES = Q3 ? 2 : 1;
  constexpr int SETS = PLANES * 2;
  const int lane = threadIdx.x & 63;
  const int b = 2 * rg + (lane >> 5), bl = lane & 31, wi = bl >> 4, jj = bl & 15, j = jj & 7;
  const int nblk = K / 32;
  const float hn = __shfl_down(h, 8, 64);     // column + 8 (used by lanes with jj < 8)
  const float hi = bf16_to_f32(f32_to_bf16_rne(h));
  const float lo = bf16_to_f32(f32_to_bf16_rne(h - hi));
  const float hin = bf16_to_f32(f32_to_bf16_rne(hn));
  const float lon = bf16_to_f32(f32_to_bf16_rne(hn - hin));
  const float sp = ldexpf(1.0f, -lo_shift(j));
  const float sq = ldexpf(4.0f, -hi_shift(j));
  if (jj < 8) {
    uint32_t* __restrict__ dst = pairs + ((size_t)row * nblk + b) * (SETS * 16) + wi * 8 + j;
    dst[0] = f32_to_bf16_rne(hi * sp) | (f32_to_bf16_rne(hin * sp) << 16);
    dst[PLANES * 16] = f32_to_bf16_rne(lo * sp) | (f32_to_bf16_rne(lon * sp) << 16);
    if (Q3) {
      dst[16] = f32_to_bf16_rne(hi * sq) | (f32_to_bf16_rne(hin * sq) << 16);
      dst[(PLANES + 1) * 16] = f32_to_bf16_rne(lo * sq) | (f32_to_bf16_rne(lon * sq) << 16);
    }
  }
  const float mult = 128.0f * sp + (Q3 ? 128.0f * sq + 4.0f : 2.0f);
  float term = mult * (hi + lo);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) term += __shfl_xor(term, off, 64);
  if (bl == 0) init[(size_t)row * nblk + b] = -term;
}

}  // namespace moe

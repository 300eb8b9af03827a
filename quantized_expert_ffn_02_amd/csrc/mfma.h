// MFMA helpers shared by the grouped GEMM kernels (gfx950, 32x32x16 f16/bf16).
//
// Fragment layouts of v_mfma_f32_32x32x16_{f16,bf16}: A: lane l holds
// A[l % 32][8 (l / 32) + j], j = 0..7; B: lane l holds B[8 (l / 32) + j][l % 32];
// C: lane l, register r holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// 2-bit weights are dequantised exactly into fp16 B fragments ("pair order"):
// inside each aligned 16-group of K the order is (0, 8, 1, 9, ..., 7, 15), the
// order in which one code word yields its pairs, and the activations are stored
// in the same order so no operand is permuted.  Lane (n, h) needs positions
// 8h .. 8h + 7 of a 16-group, the pairs (w_{4h+q}, w_{4h+q+8}), q = 0..3, whose
// codes sit at bits 2q and 16 + 2q of the code word shifted right by 8h.  OR-ing
// a code under the exponent of 1024 gives the fp16 value 1024 + c 4^q; one
// v_pk_fma_f16 turns it into c - 2 and one v_pk_mul_f16 applies the block scale,
// both exact: c - 2 in {-2, -1, 0, 1} times an fp16 scale s is an fp16 value
// as long as |s| <= 32,752 (beyond that, -2 s overflows to infinity; the
// decode kernels, which apply the scale in fp32, have no such limit).  3-bit
// weights enter as two fragments, s (lo - 2) and s (4 hi - 2) = +-2 s, with the
// same limit.
#pragma once

#include <math.h>

#include "device.h"

namespace moe {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
// native 128-bit vector (HIP's uint4 is a struct whose copies into LDS keep a
// private-memory temporary alive)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// position of column k (0..15) of a 16-group in pair order
__device__ __forceinline__ int pair_pos(int k) { return k < 8 ? 2 * k : 2 * (k - 8) + 1; }

// row (0..31) of accumulator register r for this lane, column = lane & 31
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct BConst {
  uint32_t mask[4];   // 0x00030003 << 2q
  h2_t mul[4];        // 4^-q
  h2_t add[4];        // -(1024 * 4^-q + 2)
  uint32_t magic;     // 0x64006400
};

__device__ __forceinline__ BConst bconst() {
  BConst c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c.mask[q] = vgpr_const(0x00030003u << (2 * q));
    const float m = ldexpf(1.0f, -2 * q);
    c.mul[q] = h2_t{(_Float16)m, (_Float16)m};
    const _Float16 a = (_Float16)(-(1024.0f * m + 2.0f));
    c.add[q] = h2_t{a, a};
  }
  c.magic = vgpr_const(0x64006400u);
  return c;
}

// B fragment (8 fp16 in pair order) of one lane from its code word w (already
// shifted right by 8 * lane-half) and the block scale pair s2.
__device__ __forceinline__ h8_t b_frag(uint32_t w, h2_t s2, const BConst& c) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h2_t f = __builtin_bit_cast(h2_t, (w & c.mask[q]) | c.magic);
    f = f * c.mul[q] + c.add[q];   // c - 2, exact
    f = f * s2;                    // s (c - 2), exact
    o[q] = __builtin_bit_cast(uint32_t, f);
  }
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(h8_t, u4v{o[0], o[1], o[2], o[3]});
}

// 3-bit weights, c = lo + 4 hi, w = s (c - 4) = s (lo - 2) + s (4 hi - 2): the lo
// part is the 2-bit fragment above; the hi part is a second fragment, one high
// bit per weight.  For lane (n, h) the high bits of pair q sit at bits q and
// 16 + q of the plane word shifted right by 8 (step % 2) + 4h.  Under the
// exponent of 1024 a bit gives 1024 + hi 2^q; one v_pk_fma_f16 turns that into
// 4 hi, a second one into s (4 hi - 2) = +-2s: both exact.
struct BConstHi {
  uint32_t mask[4];   // 0x00010001 << q
  h2_t mul[4];        // 4 * 2^-q
  h2_t add[4];        // -4096 * 2^-q
};

__device__ __forceinline__ BConstHi bconst_hi() {
  BConstHi c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c.mask[q] = vgpr_const(0x00010001u << q);
    const float m = ldexpf(4.0f, -q);
    c.mul[q] = h2_t{(_Float16)m, (_Float16)m};
    const _Float16 a = (_Float16)(-4096.0f * ldexpf(1.0f, -q));
    c.add[q] = h2_t{a, a};
  }
  return c;
}

// hw: the plane word shifted so that pair q's bits are at q and 16 + q;
// n2s = -2 s (both halves).
__device__ __forceinline__ h8_t b_frag_hi(uint32_t hw, h2_t s2, h2_t n2s, const BConstHi& c, uint32_t magic) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h2_t f = __builtin_bit_cast(h2_t, (hw & c.mask[q]) | magic);
    f = f * c.mul[q] + c.add[q];   // 4 hi, exact
    f = f * s2 + n2s;              // s (4 hi - 2), exact
    o[q] = __builtin_bit_cast(uint32_t, f);
  }
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(h8_t, u4v{o[0], o[1], o[2], o[3]});
}

__device__ __forceinline__ h2_t scale_pair(uint32_t d, bool hi) {
  const uint32_t v = hi ? ((d >> 16) | (d & 0xFFFF0000u)) : ((d & 0xFFFFu) | (d << 16));
  return __builtin_bit_cast(h2_t, v);
}

struct BCol {
  const u32x4* __restrict__ codes;   // this lane's column: 16 B per step
  const uint32_t* __restrict__ scales;
  const uint2* __restrict__ hi;      // 3-bit weights: the column's high bits, 8 B per step
};

// Column n of a tiled 2-bit matrix with K columns: pointer to its first 16-byte
// code chunk (steps advance by 1024 B) and to its scale dword of blocks 0, 1.
__device__ __forceinline__ BCol b_column(const uint8_t* codes, const uint16_t* scales, int n, int K,
                                        const uint8_t* hi = nullptr) {
  BCol b;
  const int nt = n >> 6, nl = n & 63;
  b.codes = reinterpret_cast<const u32x4*>(codes + ((size_t)nt * (K / 64) * 64 + nl) * 16);
  b.scales = reinterpret_cast<const uint32_t*>(scales + ((size_t)nt * (K / 128) * 64 + nl) * 4);
  b.hi = hi ? reinterpret_cast<const uint2*>(hi + ((size_t)nt * (K / 64) * 64 + nl) * 8) : nullptr;
  return b;
}

// Registers of one pipeline step: the codes + scales of the wave's two B
// columns for 64 K.
struct BRegs {
  u32x4 c0, c1;
  uint32_t s0, s1;
};

// The same for 3-bit weights: plus 8 bytes of high bits per column and step.
struct BRegs3 {
  u32x4 c0, c1;
  uint32_t s0, s1;
  uint2 h0, h1;
};

// step kc: codes at + kc * 64 uint4; scales of blocks 2kc, 2kc+1 at dword
// (kc / 2) * 128 + (kc % 2)
__device__ __forceinline__ void load_b(const BCol& b0, const BCol& b1, int kc, BRegs& R) {
  R.c0 = b0.codes[(size_t)kc * 64];
  R.s0 = b0.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
  R.c1 = b1.codes[(size_t)kc * 64];
  R.s1 = b1.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
}

__device__ __forceinline__ void load_b(const BCol& b0, const BCol& b1, int kc, BRegs3& R) {
  R.c0 = b0.codes[(size_t)kc * 64];
  R.s0 = b0.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
  R.h0 = b0.hi[(size_t)kc * 64];
  R.c1 = b1.codes[(size_t)kc * 64];
  R.s1 = b1.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
  R.h1 = b1.hi[(size_t)kc * 64];
}

// Keeps the unpacking of a B register set inside the step that consumes it:
// without this the scheduler hoists it into earlier steps, right behind the
// set's loads, and the wave waits for loads it issued two steps ahead.
__device__ __forceinline__ void pin_b(BRegs& R) {
  asm volatile("" : "+v"(R.c0), "+v"(R.c1), "+v"(R.s0), "+v"(R.s1));
}
__device__ __forceinline__ void pin_b(BRegs3& R) {
  asm volatile("" : "+v"(R.c0), "+v"(R.c1), "+v"(R.s0), "+v"(R.s1), "+v"(R.h0.x), "+v"(R.h0.y), "+v"(R.h1.x),
               "+v"(R.h1.y));
}

}  // namespace moe

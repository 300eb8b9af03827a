// Host fp32 row dots over the library's quantized tiles, one instruction set per
// build: compiled with -DMOE_HOST_ISA_NS=avx512 (AVX-512F/BW/VL/DQ) and again
// with -DMOE_HOST_ISA_NS=avx2 (AVX2 + FMA + F16C).  Written with 16-lane GCC
// vector types: one zmm register per value under AVX-512, a pair of ymm under AVX2.
//
// Weight w = s * (c - z) with the fp16 scale s of its 32-column block, c the 2-bit
// code (z = 2) or the 3-bit code lo + 4 * hi (z = 4) (the Q2_0 and IQ3 builds of
// "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU at Up to 94 Tokens/s",
// section "The numbers, measured by the author"; the tile layout is this library's,
// documented in include/moe.h).
//
// A tile row holds 64 columns in 16 code bytes; byte b carries columns 4b .. 4b+3 in
// its four 2-bit fields.  Lane b of a 16-lane vector takes byte b, and field q of
// every lane is one vector of codes for the columns 4b + q, which is why the
// activations are stored in act_pos order.  Lanes 0..7 cover the tile's first
// 32-column block and lanes 8..15 its second, so one vector of the two block
// scales (8 lanes each) applies them lane by lane; each output is the sum over
// tiles of scale * (codes . activations), reduced across the 16 lanes at the end.
#include <immintrin.h>
#include <string.h>

#include "host_tier.h"

#ifndef MOE_HOST_ISA_NS
#error "define MOE_HOST_ISA_NS (avx512 or avx2)"
#endif

namespace moe_host {
namespace MOE_HOST_ISA_NS {

typedef float v16f __attribute__((vector_size(64)));
typedef int32_t v16i __attribute__((vector_size(64)));

static inline float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static inline v16f load16(const float* p) {
  v16f v;
  memcpy(&v, p, sizeof v);
  return v;
}

// 16 code bytes widened to 16 int32 lanes (vpmovzxbd; the generic vector
// conversion compiles to byte-by-byte inserts).
static inline v16i widen_bytes(const uint8_t* p) {
#if defined(__AVX512F__)
  return (v16i)_mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)p));
#else
  const __m256i lo = _mm256_cvtepu8_epi32(_mm_loadl_epi64((const __m128i*)p));
  const __m256i hi = _mm256_cvtepu8_epi32(_mm_loadl_epi64((const __m128i*)(p + 8)));
  v16i d;
  memcpy(&d, &lo, 32);
  memcpy((char*)&d + 32, &hi, 32);
  return d;
#endif
}

// Lane sum in a fixed order (lane 0 first).
static inline float lane_sum(v16f v) {
  float s = v[0];
  for (int i = 1; i < 16; ++i) s += v[i];
  return s;
}

void prep_act_bf16(const uint16_t* x, int K, float* xp) {
  for (int k = 0; k < K; ++k) xp[act_pos(k)] = bf16_to_f32(x[k]);
}

#if defined(__AVX512F__)
// AVX-512 form: a code becomes its weight factor c - z by a table lookup instead of
// mask, subtract and convert.  vpermps reads the low 4 bits of each lane, so the
// 2-bit field shifted to the bottom (with the next field above it) indexes a table
// whose entry j is (j & 3) - 2.  For Q3 the hi bit is rotated to bit 4 of the
// index and vpermt2ps picks between two such tables ((j & 3) - 4 and (j & 3)).
template <bool Q3, int NT>
static void rows_dot_nt(const HostMat& m, int n0, int nrows, const float* const* xps, float* out, int ld) {
  const int K = m.K, KT = K / 64;
  const __m512i lane = _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  const __m512i one = _mm512_set1_epi32(1);
  const __m512i hi_base = _mm512_add_epi32(
      _mm512_add_epi32(_mm512_slli_epi32(_mm512_and_si512(_mm512_srli_epi32(lane, 2), one), 3),
                       _mm512_slli_epi32(_mm512_and_si512(_mm512_srli_epi32(lane, 1), one), 4)),
      _mm512_slli_epi32(_mm512_and_si512(lane, one), 2));
  __m512i rot[4];
  for (int q = 0; q < 4; ++q)
    rot[q] = _mm512_and_si512(_mm512_add_epi32(hi_base, _mm512_set1_epi32(q - 4)), _mm512_set1_epi32(31));
  const __m512i low2 = _mm512_set1_epi32(3);
  const __m512 tab_lo = _mm512_cvtepi32_ps(_mm512_sub_epi32(_mm512_and_si512(lane, low2), _mm512_set1_epi32(Q3 ? 4 : 2)));
  const __m512 tab_hi = _mm512_cvtepi32_ps(_mm512_and_si512(lane, low2));
  const __m512i scale_sel = _mm512_srli_epi32(lane, 3);   // 0 in lanes 0..7, 1 in 8..15
  for (int r = 0; r < nrows; ++r) {
    const int n = n0 + r;
    const size_t tile0 = (size_t)(n >> 6) * KT;
    const uint8_t* cp = m.lo + tile0 * 1024 + (size_t)(n & 63) * 16;
    const uint8_t* hp = Q3 ? m.hi + tile0 * 512 + (size_t)(n & 63) * 8 : nullptr;
    const uint16_t* sp = m.scale + (size_t)(n >> 6) * (K / 128) * 256 + (n & 63) * 4;
    __m512 acc[NT];
    for (int j = 0; j < NT; ++j) acc[j] = _mm512_setzero_ps();
    for (int kt = 0; kt < KT; ++kt) {
      // rows n .. n+3 share each 64-byte line of a tile; fetch the next four rows' line
      _mm_prefetch((const char*)(cp + (size_t)kt * 1024 + 64), _MM_HINT_T0);
      if (Q3 && (n & 7) == 0) _mm_prefetch((const char*)(hp + (size_t)kt * 512 + 64), _MM_HINT_T0);
      const __m512i d = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)(cp + (size_t)kt * 1024)));
      __m512i hv = _mm512_setzero_si512();
      if (Q3) {
        uint32_t w[2];
        memcpy(w, hp + (size_t)kt * 512, 8);
        hv = _mm512_mask_set1_epi32(_mm512_set1_epi32((int)w[1]), 0x00FF, (int)w[0]);
      }
      uint32_t sbits;
      memcpy(&sbits, sp + (kt >> 1) * 256 + (kt & 1) * 2, 4);
      const __m512 sv =
          _mm512_permutexvar_ps(scale_sel, _mm512_castps128_ps512(_mm_cvtph_ps(_mm_cvtsi32_si128((int)sbits))));
      __m512 wq[4];
      for (int q = 0; q < 4; ++q) {
        const __m512i dq = q ? _mm512_srli_epi32(d, 2 * q) : d;
        if (Q3) {
          const __m512i idx = _mm512_ternarylogic_epi32(dq, _mm512_rorv_epi32(hv, rot[q]), low2, 0xE4);
          wq[q] = _mm512_permutex2var_ps(tab_lo, idx, tab_hi);
        } else {
          wq[q] = _mm512_permutexvar_ps(dq, tab_lo);
        }
      }
      for (int j = 0; j < NT; ++j) {
        const float* xk = xps[j] + kt * 64;
        __m512 p = _mm512_mul_ps(wq[0], _mm512_loadu_ps(xk));
        p = _mm512_fmadd_ps(wq[1], _mm512_loadu_ps(xk + 16), p);
        p = _mm512_fmadd_ps(wq[2], _mm512_loadu_ps(xk + 32), p);
        p = _mm512_fmadd_ps(wq[3], _mm512_loadu_ps(xk + 48), p);
        acc[j] = _mm512_fmadd_ps(sv, p, acc[j]);
      }
    }
    for (int j = 0; j < NT; ++j) {
      v16f a;
      memcpy(&a, &acc[j], sizeof a);
      out[(size_t)r * ld + j] = lane_sum(a);
    }
  }
}
#else
// NT tokens per pass, one accumulator vector each.
template <bool Q3, int NT>
static void rows_dot_nt(const HostMat& m, int n0, int nrows, const float* const* xps, float* out, int ld) {
  const int K = m.K, KT = K / 64;
  const v16i lane = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};
  const v16i first_block = lane < 8;   // -1 in lanes 0..7
  // bit of the Q3 hi word for column 4b + q, less q: within the low 32-bit half for
  // lanes 0..7 and the high half for lanes 8..15
  const v16i hi_shift = 8 * ((lane >> 2) & 1) + 16 * ((lane >> 1) & 1) + 4 * (lane & 1);
  for (int r = 0; r < nrows; ++r) {
    const int n = n0 + r;
    const size_t tile0 = (size_t)(n >> 6) * KT;
    const uint8_t* cp = m.lo + tile0 * 1024 + (size_t)(n & 63) * 16;
    const uint8_t* hp = Q3 ? m.hi + tile0 * 512 + (size_t)(n & 63) * 8 : nullptr;
    const uint16_t* sp = m.scale + (size_t)(n >> 6) * (K / 128) * 256 + (n & 63) * 4;
    v16f acc[NT];
    for (int j = 0; j < NT; ++j) acc[j] = (v16f){};
    for (int kt = 0; kt < KT; ++kt) {
      const v16i d = widen_bytes(cp + (size_t)kt * 1024);
      v16i hv = {};
      if (Q3) {
        uint32_t w[2];
        memcpy(w, hp + (size_t)kt * 512, 8);
        const v16i w0 = (v16i){} + (int32_t)w[0], w1 = (v16i){} + (int32_t)w[1];
        hv = first_block ? w0 : w1;
      }
      const uint16_t* s2 = sp + (kt >> 1) * 256 + (kt & 1) * 2;
      const v16f s0 = (v16f){} + _cvtsh_ss(s2[0]), s1 = (v16f){} + _cvtsh_ss(s2[1]);
      const v16f sv = first_block ? s0 : s1;
      v16f cf[4];
      for (int q = 0; q < 4; ++q) {
        v16i c = (d >> (2 * q)) & 3;
        if (Q3) c |= ((hv >> (hi_shift + q)) & 1) << 2;
        cf[q] = __builtin_convertvector(c - (Q3 ? 4 : 2), v16f);
      }
      for (int j = 0; j < NT; ++j) {
        const float* xk = xps[j] + kt * 64;
        const v16f p = cf[0] * load16(xk) + cf[1] * load16(xk + 16) + cf[2] * load16(xk + 32) +
                       cf[3] * load16(xk + 48);
        acc[j] += sv * p;
      }
    }
    for (int j = 0; j < NT; ++j) out[(size_t)r * ld + j] = lane_sum(acc[j]);
  }
}
#endif

template <bool Q3>
static void rows_dot_q(const HostMat& m, int n0, int nrows, const float* const* xps, int ntok, float* out,
                       int ld) {
  constexpr int kMaxNT = 8;
  for (int t0 = 0; t0 < ntok; t0 += kMaxNT) {
    const int nt = ntok - t0 < kMaxNT ? ntok - t0 : kMaxNT;
    const float* const* xs = xps + t0;
    float* o = out + t0;
    switch (nt) {
      case 1: rows_dot_nt<Q3, 1>(m, n0, nrows, xs, o, ld); break;
      case 2: rows_dot_nt<Q3, 2>(m, n0, nrows, xs, o, ld); break;
      case 3: rows_dot_nt<Q3, 3>(m, n0, nrows, xs, o, ld); break;
      case 4: rows_dot_nt<Q3, 4>(m, n0, nrows, xs, o, ld); break;
      case 5: rows_dot_nt<Q3, 5>(m, n0, nrows, xs, o, ld); break;
      case 6: rows_dot_nt<Q3, 6>(m, n0, nrows, xs, o, ld); break;
      case 7: rows_dot_nt<Q3, 7>(m, n0, nrows, xs, o, ld); break;
      default: rows_dot_nt<Q3, 8>(m, n0, nrows, xs, o, ld); break;
    }
  }
}

void rows_dot(const HostMat& m, int n0, int nrows, const float* const* xps, int ntok, float* out, int ld) {
  if (m.hi)
    rows_dot_q<true>(m, n0, nrows, xps, ntok, out, ld);
  else
    rows_dot_q<false>(m, n0, nrows, xps, ntok, out, ld);
}

}  // namespace MOE_HOST_ISA_NS
}  // namespace moe_host

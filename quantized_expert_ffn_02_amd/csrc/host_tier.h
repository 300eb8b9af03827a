// Host (CPU) side of the expert tiers: the experts a GPU cache does not hold are
// computed by the host's cores from a copy of every expert kept in system memory,
// while the GPU computes the cached ones ("Strata Runs 125B Qwen3.8-Flash-Next on a
// 12GB Gaming GPU at Up to 94 Tokens/s", section "How a 125B model fits in 12 GB";
// the aireport.net page names AVX-512 and AVX2 kernels for this part).
//
// The arithmetic is fp32 on the vector units.  The routines that depend on the
// instruction set live in host_ffn.cpp, which is compiled twice (AVX-512 and
// AVX2 + FMA) into the namespaces declared below; host_tier.cpp picks one at run
// time and holds the rest (grouping, SiLU, fixed-order sums, the thread pool).
#pragma once
#include <stdint.h>

namespace moe_host {

// One quantized matrix of the library's tiled layout (see include/moe.h): N rows,
// K columns, Q2 codes (hi == nullptr) or Q3 (lo + hi planes), fp16 block scales.
struct HostMat {
  const uint8_t* lo;
  const uint8_t* hi;
  const uint16_t* scale;
  int N, K;
};

// Activations of one token in the order the row dot reads them: for each 64-column
// tile kt, value x[kt*64 + 4b + q] is stored at kt*64 + 16q + b (b 0..15, q 0..3),
// so that the q-th 2-bit field of the b-th code byte of a tile row meets it in lane b.
inline int act_pos(int k) { return (k & ~63) + ((k & 3) << 4) + ((k & 63) >> 2); }

#define MOE_HOST_ISA_DECL(ns)                                                              \
  namespace ns {                                                                           \
  /* xp[act_pos(k)] = float(bf16 x[k]) for k < K */                                        \
  void prep_act_bf16(const uint16_t* x, int K, float* xp);                                 \
  /* out[r * ld + j] = sum_k W[n0 + r, k] * act_j[k] for r < nrows, j < ntok, with         \
     W dequantised as s * (c - z); act_j given in act_pos order (xps[j]). */               \
  void rows_dot(const HostMat& m, int n0, int nrows, const float* const* xps, int ntok,     \
                float* out, int ld);                                                        \
  }

MOE_HOST_ISA_DECL(avx512)
MOE_HOST_ISA_DECL(avx2)
#undef MOE_HOST_ISA_DECL

}  // namespace moe_host

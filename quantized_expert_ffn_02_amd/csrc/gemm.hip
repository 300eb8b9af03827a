// MFMA grouped GEMMs for prefill chunks and large token groups, and the MFMA
// router GEMM.
//
// A prompt is read in chunks of up to 8,192 tokens (page "Strata Runs a
// 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU at up to 93 Tokens per
// Second"); for such a chunk every expert that a few dozen or more tokens chose
// is a dense [M_e x 2560] x [2560 x 1280] product followed by [M_e x 640] x
// [640 x 2560], which belongs on the matrix cores.
//
// Precision: the weights are dequantised EXACTLY into fp16 (s * (c - 2) with an
// fp16 scale and c - 2 in {-2, -1, 0, 1} is an fp16 value), activations enter as
// fp16 (bf16 -> fp16 is exact for |x| >= 2^-17 and below 65504), products are
// exact and accumulate in fp32 (v_mfma_f32_32x32x16_f16); h = SiLU(gate) * up is
// carried in fp16 between the two GEMMs and the output is fp32.
//
// Operand order: the 2-bit unpacking yields weights in "pair order" -- inside
// each aligned group of 16 columns the order is (0, 8, 1, 9, ..., 7, 15).  The
// MFMA sums over K in any order as long as both operands agree, so the fp16
// activations (x, and h from the gate/up epilogue) are stored in the same order
// and no operand is ever permuted inside the GEMM.
//
// Tiles: a block computes 128 rows (sorted positions of one expert) x 128
// columns with 4 waves of 64 x 64 (2 x 2 MFMA 32x32 tiles); the K loop steps by
// 64 with double-buffered LDS: the next step's global loads are in flight while
// the current step's MFMAs run, and the dequantisation happens on the way into
// LDS.  The gate/up kernel's 128 columns are 64 gate + the 64 matching up
// columns, so SwiGLU is applied in registers.
#include <math.h>

#include "device.h"
#include "internal.h"

namespace moe {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
// native 128-bit vector (HIP's uint4 is a struct whose copies into LDS keep a
// private-memory temporary alive)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int LDS_STRIDE = BK + 8;   // halves per LDS row (padding against bank conflicts)

// position of column k (0..15) of a 16-group in pair order
__device__ __forceinline__ int pair_pos(int k) { return k < 8 ? 2 * k : 2 * (k - 8) + 1; }

// ---------------------------------------------------------------------------
// x (bf16) -> fp16 in pair order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_x_to_f16_pairs(const uint16_t* __restrict__ x, size_t n16,
                                                        uint16_t* __restrict__ out) {
  // one thread per 16-group
  for (size_t g = (size_t)blockIdx.x * 256 + threadIdx.x; g < n16; g += (size_t)gridDim.x * 256) {
    const uint4* src = reinterpret_cast<const uint4*>(x + g * 16);
    const uint4 a = src[0], b = src[1];
    const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column j (low half of in[j/2] if j even) and column j + 8
      const uint32_t v0 = (j & 1) ? (in[j >> 1] >> 16) : (in[j >> 1] & 0xFFFFu);
      const uint32_t v1 = (j & 1) ? (in[4 + (j >> 1)] >> 16) : (in[4 + (j >> 1)] & 0xFFFFu);
      const _Float16 f0 = (_Float16)bf16_to_f32(v0), f1 = (_Float16)bf16_to_f32(v1);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, f0) | ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + g * 16);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

hipError_t launch_x_to_f16_pairs(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s) {
  const size_t n16 = (size_t)T * H / 16;
  const int blocks = (int)((n16 + 255) / 256 < 2048 ? (n16 + 255) / 256 : 2048);
  MOE_LAUNCH(k_x_to_f16_pairs, dim3(blocks), dim3(256), 0, s, x, n16, out);
  return hipGetLastError();
}

// row (0..31) of accumulator register r for this lane, column = lane & 31
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// Grouped GEMM over the 2-bit experts.
//
// A block owns one M-tile (up to GBM = 128 sorted rows of one expert group) and
// 4 x 64 weight rows ("columns" of the product); each of its 4 waves computes
// all 128 rows x its own 64 columns as 4 x 2 MFMA 32x32x16 tiles.  The
// activations A are shared by the 4 waves and go through LDS (double-buffered,
// rows padded to 72 halves so that the fragment reads are free of bank
// conflicts).  The weights B are used by exactly one wave, so each wave reads
// its 2-bit codes straight from global memory into registers and dequantises
// them there into MFMA B fragments: no LDS traffic and no duplicated work for B.
//
// B fragment of a 32x32x16 MFMA: lane l holds 8 consecutive K positions
// 8 (l / 32) .. + 7 of column l % 32.  In pair order, positions 8h .. 8h + 7 of
// a 16-group are the pairs (w_{4h+q}, w_{4h+q+8}), q = 0..3, whose codes sit at
// bits 2q and 16 + 2q of the code word shifted right by 8h.  OR-ing a code under
// the exponent of 1024 gives the fp16 value 1024 + c 4^q; one v_pk_fma_f16 turns
// it into c - 2 (exact) and one v_pk_mul_f16 applies the block scale (exact).
// ---------------------------------------------------------------------------
static constexpr int GBM = 128;              // rows per M-tile
static constexpr int GBK = 64;               // K per pipeline step
static constexpr int A_STRIDE = GBK + 8;     // halves per LDS row
static constexpr int GCOLS = 256;            // weight rows per block (4 waves x 64)

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

__device__ __forceinline__ h2_t scale_pair(uint32_t d, bool hi) {
  const uint32_t v = hi ? ((d >> 16) | (d & 0xFFFF0000u)) : ((d & 0xFFFFu) | (d << 16));
  return __builtin_bit_cast(h2_t, v);
}

// Registers of one pipeline step: 64 K of A for this thread's LDS row slice and
// the codes + scales of the wave's two B columns.
struct StepRegs {
  u32x4 a0, a1, a2, a3;
  u32x4 c0, c1;
  uint32_t s0, s1;
};

struct BCol {
  const u32x4* __restrict__ codes;   // this lane's column: 16 B per step
  const uint32_t* __restrict__ scales;
};

// Column n of a tiled 2-bit matrix with K columns: pointer to its first 16-byte
// code chunk (steps advance by 1024 B) and to its scale dword of blocks 0, 1.
__device__ __forceinline__ BCol b_column(const uint8_t* codes, const uint16_t* scales, int n, int K) {
  BCol b;
  const int nt = n >> 6, nl = n & 63;
  b.codes = reinterpret_cast<const u32x4*>(codes + ((size_t)nt * (K / 64) * 64 + nl) * 16);
  b.scales = reinterpret_cast<const uint32_t*>(scales + ((size_t)nt * (K / 128) * 64 + nl) * 4);
  return b;
}

// step kc: codes at + kc * 64 uint4; scales of blocks 2kc, 2kc+1 at dword
// (kc / 2) * 128 + (kc % 2)
__device__ __forceinline__ void load_b(const BCol& b, int kc, u32x4& c, uint32_t& s) {
  c = b.codes[(size_t)kc * 64];
  s = b.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
}

// One K step of a wave: 4 x (2 B fragments, 4 A fragments, 8 MFMAs).
__device__ __forceinline__ void wave_step(const uint16_t* __restrict__ As, const StepRegs& R, int shift,
                                          const BConst& bc, f16x_t acc[4][2]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const uint32_t cw0[4] = {R.c0.x, R.c0.y, R.c0.z, R.c0.w};
  const uint32_t cw1[4] = {R.c1.x, R.c1.y, R.c1.z, R.c1.w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const h8_t b0 = b_frag(cw0[s] >> shift, scale_pair(R.s0, s >= 2), bc);
    const h8_t b1 = b_frag(cw1[s] >> shift, scale_pair(R.s1, s >= 2), bc);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const h8_t a = *reinterpret_cast<const h8_t*>(As + (mi * 32 + r) * A_STRIDE + s * 16 + kh);
      acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc[mi][0], 0, 0, 0);
      acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc[mi][1], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM tiles: (group, first sorted position, rows <= GBM) per M-tile.
// ---------------------------------------------------------------------------
struct GemmTile {
  int g, m0, rows, n;   // n = column-tile index
};

// Workgroups are placed on the 8 XCDs round-robin by linear id.  Only the
// first n_valid = tiles x column-tiles linear ids carry work (the grid is a host
// bound); re-number those so that XCD x runs a contiguous range of logical
// tiles, column-tile fastest: the column tiles of one row tile then share its
// activation rows in one L2, and every XCD still gets 1/8 of the work.
__device__ __forceinline__ int xcd_logical_id(int lin, int n_valid) {
  const int per = (n_valid + 7) / 8;
  const int xcd = lin & 7, slot = lin >> 3;
  const int full = n_valid - 8 * (per - 1);   // XCDs that get `per` ids (the rest get per - 1)
  return xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
}

__device__ __forceinline__ bool load_tile(const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
                                          GemmTile& t) {
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int n_valid = n_tiles[0] * (int)gridDim.y;
  if (lin >= n_valid) return false;
  const int id = xcd_logical_id(lin, n_valid);
  const int mt = id / gridDim.y;
  t.n = id % gridDim.y;
  t.g = tiles[3 * mt];
  t.m0 = tiles[3 * mt + 1];
  t.rows = tiles[3 * mt + 2];
  return true;
}

// ---------------------------------------------------------------------------
// The grouped GEMM kernel for both projections.
//   GateUp: rows p of the tile are tokens t(p) (x_f16 rows), K = H; wave w of
//           column tile j owns gate rows 128 j + 32 w + (0..31) and the same up
//           rows; the epilogue writes h = SiLU(gate) * up in fp16, pair order.
//   Down:   rows p are rows of h (K = I); wave w of column tile j owns output
//           columns 256 j + 64 w + (0..63); the epilogue writes fp32 y.
// K / 64 (the number of steps) is even: H and I are multiples of 128.
// ---------------------------------------------------------------------------
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_gemm_q2(
    const uint8_t* __restrict__ r_codes, const uint16_t* __restrict__ r_scales, const uint8_t* __restrict__ s_codes,
    const uint16_t* __restrict__ s_scales, size_t code_stride, size_t scale_stride, int H, int I, int E,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ sorted_rows,
    int T, int k, const uint16_t* __restrict__ a_src, uint16_t* __restrict__ h_out, float* __restrict__ y_out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * A_STRIDE];
  GemmTile t;
  if (!load_tile(tiles, n_tiles, t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool sh = t.g == E;
  const size_t eidx = sh ? 0 : (size_t)t.g;
  const uint8_t* codes = (sh ? s_codes : r_codes) + eidx * code_stride;
  const uint16_t* scales = (sh ? s_scales : r_scales) + eidx * scale_stride;
  const int K = GATEUP ? H : I;
  const int nch = K / GBK;

  // A staging: thread -> (row ra = tid / 2, 32-half slice ha = tid % 2) of the step
  const int ra = tid >> 1, ha = tid & 1;
  const int pa = t.m0 + (ra < t.rows ? ra : 0);
  size_t arow;
  if (GATEUP) {
    const int r = sorted_rows[pa];
    const int Tk = T * k;
    arow = (size_t)(r < Tk ? r / k : r - Tk);
  } else {
    arow = (size_t)pa;
  }
  const u32x4* __restrict__ ag = reinterpret_cast<const u32x4*>(a_src + arow * K) + ha * 4;
  uint16_t* const as_dst0 = &As[0][ra * A_STRIDE + ha * 32];
  uint16_t* const as_dst1 = &As[1][ra * A_STRIDE + ha * 32];

  // B columns of this lane
  int n0, n1;
  if (GATEUP) {
    n0 = t.n * 128 + wv * 32 + (lane & 31);
    n1 = I + n0;
  } else {
    n0 = t.n * GCOLS + wv * 64 + (lane & 31);
    n1 = n0 + 32;
  }
  const BCol B0 = b_column(codes, scales, n0, K);
  const BCol B1 = b_column(codes, scales, n1, K);
  const int shift = (lane >> 5) * 8;
  const BConst bc = bconst();

  f16x_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto load_step = [&](StepRegs& R, int kc) {
    R.a0 = ag[kc * 8 + 0];
    R.a1 = ag[kc * 8 + 1];
    R.a2 = ag[kc * 8 + 2];
    R.a3 = ag[kc * 8 + 3];
    load_b(B0, kc, R.c0, R.s0);
    load_b(B1, kc, R.c1, R.s1);
  };
  auto store_a = [&](const StepRegs& R, uint16_t* dst) {
    u32x4* d = reinterpret_cast<u32x4*>(dst);
    d[0] = R.a0;
    d[1] = R.a1;
    d[2] = R.a2;
    d[3] = R.a3;
  };

  // Two register sets; the loop is unrolled by two so both keep static names.
  // Step kc computes from LDS buffer kc % 2 and register set kc % 2 while the
  // loads of step kc + 1 (other set) are in flight.
  StepRegs R0, R1;
  load_step(R0, 0);
  store_a(R0, as_dst0);
  __syncthreads();
  for (int kc = 0; kc < nch; kc += 2) {
    load_step(R1, kc + 1);
    wave_step(As[0], R0, shift, bc, acc);
    store_a(R1, as_dst1);
    __syncthreads();
    if (kc + 2 < nch) load_step(R0, kc + 2);
    wave_step(As[1], R1, shift, bc, acc);
    if (kc + 2 < nch) store_a(R0, as_dst0);
    __syncthreads();
  }

  if (GATEUP) {
    // h = SiLU(gate) * up, fp16, stored at the pair-order position of its column
    const int col = t.n * 128 + wv * 32 + (lane & 31);
    const int pcol = (col & ~15) + pair_pos(col & 15);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mi * 32 + acc_row(r, lane);
        if (row < t.rows) {
          const float g = acc[mi][0][r], u = acc[mi][1][r];
          const float hv = g / (1.0f + expf(-g)) * u;
          h_out[(size_t)(t.m0 + row) * I + pcol] = __builtin_bit_cast(uint16_t, (_Float16)hv);
        }
      }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + acc_row(r, lane);
          if (row < t.rows) y_out[(size_t)(t.m0 + row) * H + (f ? n1 : n0)] = acc[mi][f][r];
        }
  }
}

hipError_t launch_gemm_q2(GemvKind kind, const MatRef& routed, const MatRef& shared, int H, int I, int E,
                          const int32_t* tiles, const int32_t* n_tiles, int max_tiles, const int32_t* sorted_rows,
                          int T, int k, const uint16_t* a_f16, void* out, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (kind == GemvKind::GateUp) {
    MOE_LAUNCH(k_gemm_q2<true>, dim3(max_tiles, I / 128), dim3(256), 0, s, routed.codes, routed.scales,
                       shared.codes, shared.scales, routed.code_stride, routed.scale_stride, H, I, E, tiles, n_tiles,
                       sorted_rows, T, k, a_f16, (uint16_t*)out, nullptr);
  } else {
    MOE_LAUNCH(k_gemm_q2<false>, dim3(max_tiles, H / GCOLS), dim3(256), 0, s, routed.codes, routed.scales,
                       shared.codes, shared.scales, routed.code_stride, routed.scale_stride, H, I, E, tiles, n_tiles,
                       nullptr, T, k, a_f16, nullptr, (float*)out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router GEMM (bf16 MFMA): logits[t, e] = x_t . Wr[e] + b[e] for 128 x 128 tiles.
// Both operands are bf16 in natural column order; products are exact in fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ b8_t lds_frag_b(const uint16_t* base, int row, int k) {
  return *reinterpret_cast<const b8_t*>(base + row * LDS_STRIDE + k);
}

__global__ __launch_bounds__(256, 2) void k_router_mfma(const uint16_t* __restrict__ x, int T,
                                                        const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ bias, int E, int H,
                                                        float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int ra = tid >> 1, ha = tid & 1;
  const int arow_i = min(m0 + ra, T - 1), brow_i = min(n0 + ra, E - 1);
  const u32x4* __restrict__ arow = reinterpret_cast<const u32x4*>(x + (size_t)arow_i * H) + ha * 4;
  const u32x4* __restrict__ brow = reinterpret_cast<const u32x4*>(wr + (size_t)brow_i * H) + ha * 4;
  const int nch = H / 64;
  u32x4 pa[4], pb[4];
  auto load_step = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa[q] = arow[kc * 8 + q];
      pb[q] = brow[kc * 8 + q];
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      reinterpret_cast<u32x4*>(&As[buf][ra * LDS_STRIDE + ha * 32])[q] = pa[q];
      reinterpret_cast<u32x4*>(&Bs[buf][ra * LDS_STRIDE + ha * 32])[q] = pb[q];
    }
  };
  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int a0 = (wv >> 1) * 64, b0 = (wv & 1) * 64;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int kc = 0; kc < nch; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nch) load_step(kc + 1);
#pragma unroll
    for (int k16 = 0; k16 < BK; k16 += 16) {
      const b8_t fa0 = lds_frag_b(As[buf], a0 + r32, k16 + kh);
      const b8_t fa1 = lds_frag_b(As[buf], a0 + 32 + r32, k16 + kh);
      const b8_t fb0 = lds_frag_b(Bs[buf], b0 + r32, k16 + kh);
      const b8_t fb1 = lds_frag_b(Bs[buf], b0 + 32 + r32, k16 + kh);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb1, acc[1][1], 0, 0, 0);
    }
    if (kc + 1 < nch) store_step(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + a0 + 32 * mi + acc_row(r, lane);
        const int col = n0 + b0 + 32 * ni + r32;
        if (row < T && col < E) logits[(size_t)row * E + col] = acc[mi][ni][r] + (bias ? bias[col] : 0.0f);
      }
}

hipError_t launch_router_mfma(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s) {
  dim3 grid((T + BM - 1) / BM, (E + BN - 1) / BN);
  MOE_LAUNCH(k_router_mfma, grid, dim3(256), 0, s, x, T, wr, bias, E, H, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: split the groups of a permutation between the MFMA GEMM (groups with at
// least min_rows entries, cut into BM-row tiles) and the GEMV work items (the
// rest, items_per entries each).  One block of 1024 threads, thread = group.
// ---------------------------------------------------------------------------
__device__ int plan_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    const int s = wsum[i];
    if (i < w) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ offsets, int E, int min_rows,
                                               int items_per, int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ n_tiles, int32_t* __restrict__ items,
                                               int32_t* __restrict__ n_items) {
  const int G = E + 1;
  const int g = threadIdx.x;
  const int start = g < G ? offsets[g] : 0;
  const int cnt = g < G ? offsets[g + 1] - start : 0;
  const bool big = cnt >= min_rows;
  const int nt = big ? (cnt + BM - 1) / BM : 0;
  const int ni = big ? 0 : (cnt + items_per - 1) / items_per;
  int tot_t = 0, tot_i = 0;
  const int pt = plan_scan_1024(nt, &tot_t);
  const int pi = plan_scan_1024(ni, &tot_i);
  for (int i = 0; i < nt; ++i) {
    tiles[3 * (pt + i)] = g;
    tiles[3 * (pt + i) + 1] = start + i * BM;
    tiles[3 * (pt + i) + 2] = min(BM, cnt - i * BM);
  }
  for (int i = 0; i < ni; ++i) {
    items[3 * (pi + i)] = g;
    items[3 * (pi + i) + 1] = start + i * items_per;
    items[3 * (pi + i) + 2] = min(items_per, cnt - i * items_per);
  }
  if (g == 0) {
    *n_tiles = tot_t;
    *n_items = tot_i;
  }
}

hipError_t launch_plan(const int32_t* offsets, int E, int min_rows, int items_per, int32_t* tiles,
                       int32_t* n_tiles, int32_t* items, int32_t* n_items, hipStream_t s) {
  MOE_LAUNCH(k_plan, dim3(1), dim3(1024), 0, s, offsets, E, min_rows, items_per, tiles, n_tiles, items,
                     n_items);
  return hipGetLastError();
}

int gemm_tile_rows() { return GBM; }
bool gemm_shape_ok(int H, int I) { return H % GCOLS == 0 && I % 128 == 0; }

}  // namespace moe

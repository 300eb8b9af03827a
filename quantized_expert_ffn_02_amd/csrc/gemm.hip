// MFMA grouped GEMMs over the quantized experts, and the MFMA router GEMM of
// prompt chunks.
//
// A prompt is read in chunks of up to 8,192 tokens (page "Strata Runs a
// 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU at up to 93 Tokens per
// Second"); for such a chunk, and for verify batches of many sequences, every
// expert chosen by a few or more tokens is a dense [M_e x 2560] x [2560 x 1280]
// product followed by [M_e x 640] x [640 x 2560], which belongs on the matrix
// cores.
//
// Precision: the weights are dequantised EXACTLY into fp16 (mfma.h: s (c - 2)
// with an fp16 scale and c - 2 in {-2, -1, 0, 1} is an fp16 value; 3-bit
// weights as two exact fragments), activations enter as fp16 after a per-row
// power-of-two scale (k_x_to_f16_rows: every bf16 value of at least 2^-17 of
// its row's largest magnitude converts exactly, whatever that magnitude),
// products are exact and accumulate in fp32 (v_mfma_f32_32x32x16_f16); h =
// SiLU(gate) * up is carried in fp16 between the two GEMMs, in the row's
// scale (h 4^a).  The down projection writes fp32 rows with the scale undone,
// or, for a prompt chunk, fp16 rows in the row's scale already multiplied by
// their gate (the combine undoes the scale).
//
// Operand order: the 2-bit unpacking yields weights in "pair order" -- inside
// each aligned group of 16 columns the order is (0, 8, 1, 9, ..., 7, 15).  The
// MFMA sums over K in any order as long as both operands agree, so the fp16
// activations (x, and h from the gate/up epilogue) are stored in the same order
// and no operand is ever permuted inside the GEMM.
#include <math.h>

#include <type_traits>

#include "device.h"
#include "internal.h"
#include "mfma.h"
#include "mx_group.h"

namespace moe {

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int LDS_STRIDE = BK + 8;   // halves per LDS row (padding against bank conflicts)

// ---------------------------------------------------------------------------
// x (bf16) -> fp16 in pair order, each row scaled by a power of two.
//
// fp16 holds a bf16 value exactly only between about 2^-17 and 65,504, so a
// row is first scaled by 2^a, a = -floor(log2 max|x_row|): its largest
// magnitude lands in [1, 2) and every element of at least 2^-17 of it converts
// exactly (the rest are below the fp16 grid's 2^-25 rounding, far under the
// products that matter).  The GEMMs work on x' = x 2^a and undo the scale in
// fp32 (exact: a power of two): gate/up writes h' = g' u' sigma(g' 2^-a) =
// h 4^a, the down projection y 4^-a.  Zero, inf or NaN maxima give a = 0.
// One block of 256 threads per row: the row's largest magnitude from its bit
// patterns (|x| orders as the low 15 bits of a finite bf16), then the scaled
// conversion (the second read hits the cache).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_x_to_f16_rows(const uint16_t* __restrict__ x, int H,
                                                       uint16_t* __restrict__ out, int32_t* __restrict__ xexp) {
  __shared__ uint32_t wmax[4];
  const int row = blockIdx.x, n16 = H / 16;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)row * H);
  uint32_t m = 0;
  for (int g = threadIdx.x; g < n16; g += 256) {
    const uint4 a = src[2 * g], b = src[2 * g + 1];
    const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, max(in[j] & 0x7FFFu, (in[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int a = bf16_row_exponent(m);
  if (threadIdx.x == 0) xexp[row] = a;
  uint4* dst = reinterpret_cast<uint4*>(out + (size_t)row * H);
  for (int g = threadIdx.x; g < n16; g += 256) {
    const uint4 va = src[2 * g], vb = src[2 * g + 1];
    const uint32_t in[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column j (low half of in[j/2] if j even) and column j + 8
      const uint32_t v0 = (j & 1) ? (in[j >> 1] >> 16) : (in[j >> 1] & 0xFFFFu);
      const uint32_t v1 = (j & 1) ? (in[4 + (j >> 1)] >> 16) : (in[4 + (j >> 1)] & 0xFFFFu);
      const _Float16 f0 = (_Float16)ldexpf(bf16_to_f32(v0), a), f1 = (_Float16)ldexpf(bf16_to_f32(v1), a);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, f0) | ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
    }
    dst[2 * g] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[2 * g + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

hipError_t launch_x_to_f16_pairs(const uint16_t* x, int T, int H, uint16_t* out, int32_t* xexp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  MOE_LAUNCH(k_x_to_f16_rows, dim3(T), dim3(256), 0, s, x, H, out, xexp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM over the quantized experts.
//
// A block owns one M-tile (up to 128 or 32 sorted rows of one expert group) and
// 4 x 64 weight rows ("columns" of the product); each of its 4 waves computes
// all the tile's rows x its own 64 columns as 32x32x16 MFMA tiles.  The
// activations A are shared by the 4 waves and go through LDS (three buffers,
// rows padded to 72 halves so that the fragment reads are free of bank
// conflicts).  The weights B are used by exactly one wave, so each wave reads
// its codes straight from global memory into registers and dequantises them
// there into MFMA B fragments (mfma.h): no LDS traffic and no duplicated work
// for B.  Loads run DEPTH K-steps ahead through rings of register sets.
// ---------------------------------------------------------------------------
static constexpr int GBM = 128;              // rows per M-tile (32 x fragments per wave)
static constexpr int GBK = 64;               // K per pipeline step
static constexpr int A_STRIDE = GBK + 8;     // halves per LDS row
static constexpr int GCOLS = 256;            // weight rows per block (4 waves x 64)

// One K step of a wave: 4 x (2 B fragments, NMI A fragments, 2 NMI MFMAs);
// NMI = number of 32-row fragments the tile's rows need.  3-bit weights add the
// high-bit fragment of each column and a second MFMA into the same accumulator.
//
// TR (128-row tiles): the weights enter as the MFMA's first operand and the
// activations as its second, so the accumulator holds C^T: lane l has token
// row 32 mi + l % 32 and, in registers 4 q .. 4 q + 3, four consecutive output
// columns 8 q + 4 (l / 32) + (0..3) -- the epilogue stores rows in 8- and
// 16-byte pieces instead of 2-byte scatters.
// h' = h 4^a from the accumulators g' = g 2^a, u' = u 2^a of a row scaled by 2^a:
// SiLU(g) u 4^a = g' u' sigma(g), with g = g' 2^-a formed only inside sigma
// (which saturates), so h' stays finite whatever the scale of x.  sigma takes the
// hardware exponential and reciprocal (a few ulp of fp32, against the 2^-11 of the
// fp16 that h is rounded to next) instead of an IEEE division sequence.
__device__ __forceinline__ float swiglu_scaled(float gv, float uv, int a) {
  return gv * uv * __builtin_amdgcn_rcpf(1.0f + __expf(-ldexpf(gv, -a)));
}

template <bool TR>
__device__ __forceinline__ f16x_t mfma_op(h8_t a, h8_t b, f16x_t c) {
  return TR ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0)
            : __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int NMI, int MAXNMI, bool Q3, bool TR, typename BR>
__device__ __forceinline__ void wave_step(const uint16_t* __restrict__ As, const BR& R, int shift, int hshift,
                                          const BConst& bc, const BConstHi& bch, f16x_t acc[MAXNMI][2]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const uint32_t cw0[4] = {R.c0.x, R.c0.y, R.c0.z, R.c0.w};
  const uint32_t cw1[4] = {R.c1.x, R.c1.y, R.c1.z, R.c1.w};
  if constexpr (TR && !Q3) {
    // Software pipeline over the 4 sub-steps: the dequant of sub-step s + 1
    // is scheduled in slices between the MFMAs of sub-step s (scheduling
    // groups: the A reads, then per MFMA a few VALU instructions), so the
    // matrix core and the VALU work side by side within the wave.
    h8_t c0 = b_frag(cw0[0] >> shift, scale_pair(R.s0, false), bc);
    h8_t c1 = b_frag(cw1[0] >> shift, scale_pair(R.s1, false), bc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8_t a[NMI];
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) a[mi] = *reinterpret_cast<const h8_t*>(As + (mi * 32 + r) * A_STRIDE + s * 16 + kh);
      h8_t n0 = c0, n1 = c1;
      if (s < 3) {
        n0 = b_frag(cw0[s + 1] >> shift, scale_pair(R.s0, s + 1 >= 2), bc);
        n1 = b_frag(cw1[s + 1] >> shift, scale_pair(R.s1, s + 1 >= 2), bc);
      }
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) {
        acc[mi][0] = mfma_op<TR>(a[mi], c0, acc[mi][0]);
        acc[mi][1] = mfma_op<TR>(a[mi], c1, acc[mi][1]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NMI, 0);   // LDS reads
#pragma unroll
      for (int j = 0; j < 2 * NMI; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (s < 3) __builtin_amdgcn_sched_group_barrier(0x002, (28 + 2 * NMI - 1) / (2 * NMI), 0);   // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      c0 = n0;
      c1 = n1;
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const h2_t s20 = scale_pair(R.s0, s >= 2), s21 = scale_pair(R.s1, s >= 2);
    const h8_t b0 = b_frag(cw0[s] >> shift, s20, bc);
    const h8_t b1 = b_frag(cw1[s] >> shift, s21, bc);
    h8_t bh0, bh1;
    if constexpr (Q3) {
      const h2_t m2 = h2_t{(_Float16)-2.0f, (_Float16)-2.0f};
      const int hs = hshift + 8 * (s & 1);
      bh0 = b_frag_hi((s < 2 ? R.h0.x : R.h0.y) >> hs, s20, s20 * m2, bch, bc.magic);
      bh1 = b_frag_hi((s < 2 ? R.h1.x : R.h1.y) >> hs, s21, s21 * m2, bch, bc.magic);
    }
#pragma unroll
    for (int mi = 0; mi < NMI; ++mi) {
      const h8_t a = *reinterpret_cast<const h8_t*>(As + (mi * 32 + r) * A_STRIDE + s * 16 + kh);
      acc[mi][0] = mfma_op<TR>(a, b0, acc[mi][0]);
      acc[mi][1] = mfma_op<TR>(a, b1, acc[mi][1]);
      if constexpr (Q3) {
        acc[mi][0] = mfma_op<TR>(a, bh0, acc[mi][0]);
        acc[mi][1] = mfma_op<TR>(a, bh1, acc[mi][1]);
      }
    }
  }
}

// Half-width 32-row tiles (3-bit): the wave's one 32-column B fragment for a
// 64-K step -- its codes, high bits and scales -- as two exact fragments and two
// MFMAs into one accumulator per 16 K.
struct BRegsH3 {
  u32x4 c0;
  uint32_t s0;
  uint2 h0;
};
__device__ __forceinline__ void pin_b(BRegsH3& R) {
  asm volatile("" : "+v"(R.c0), "+v"(R.s0), "+v"(R.h0.x), "+v"(R.h0.y));
}

__device__ __forceinline__ void wave_step_half3(const uint16_t* __restrict__ As, const BRegsH3& R, int shift,
                                                int hshift, const BConst& bc, const BConstHi& bch, f16x_t& acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const uint32_t cw[4] = {R.c0.x, R.c0.y, R.c0.z, R.c0.w};
  const h2_t m2 = h2_t{(_Float16)-2.0f, (_Float16)-2.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const h2_t s2 = scale_pair(R.s0, s >= 2);
    const h8_t b = b_frag(cw[s] >> shift, s2, bc);
    const h8_t bh = b_frag_hi((s < 2 ? R.h0.x : R.h0.y) >> (hshift + 8 * (s & 1)), s2, s2 * m2, bch, bc.magic);
    const h8_t a = *reinterpret_cast<const h8_t*>(As + r * A_STRIDE + s * 16 + kh);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bh, acc, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM tiles: (group, first sorted position, rows <= GBM) per M-tile.
// ---------------------------------------------------------------------------
struct GemmTile {
  int g, m0, rows, n;   // n = column-tile index
  bool mx;              // a small group on the fp8 x fp4 matrix cores (mx_group.h)
};

// Workgroups are placed on the 8 XCDs round-robin by linear id.  Only the
// first n_valid = tiles x column-tiles linear ids carry work (the grid is a host
// bound); re-number those so that XCD x runs a contiguous range of logical
// tiles, column-tile fastest: the column tiles of one row tile then share its
// activation rows in one L2, and every XCD still gets 1/8 of the work.  The
// fp16 tiles, listed first by the plan, are numbered apart from the fp8 x fp4
// tiles after them, so that every XCD starts with its share of the longer ones.
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
  const int n_f16 = n_tiles[1] * (int)gridDim.y;
  const int id = lin < n_f16 ? xcd_logical_id(lin, n_f16) : n_f16 + xcd_logical_id(lin - n_f16, n_valid - n_f16);
  const int mt = id / gridDim.y;
  t.n = id % gridDim.y;
  t.g = tiles[3 * mt];
  t.m0 = tiles[3 * mt + 1];
  const int rw = tiles[3 * mt + 2];
  t.rows = rw & (kTileMx - 1);
  t.mx = (rw & kTileMx) != 0;
  return true;
}

// ---------------------------------------------------------------------------
// The grouped GEMM kernel for both projections.
//   GateUp: rows p of the tile are tokens t(p) (x_f16 rows), K = H; wave w of
//           column tile j owns gate rows 128 j + 32 w + (0..31) and the same up
//           rows; the epilogue writes h = SiLU(gate) * up in fp16, pair order.
//   Down:   rows p are rows of h (K = I); wave w of column tile j owns output
//           columns 256 j + 64 w + (0..63); the epilogue writes fp32 y.
// Pipeline: A (shared through three LDS buffers) and the wave's B codes are both
// loaded two steps ahead of their use.  A tile of fewer than 128 rows runs
// only the 32-row fragments it needs (NMI = ceil(rows / 32)).
// ---------------------------------------------------------------------------
struct GemmArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* hi;      // 3-bit weights: high-bit plane
  int H, I, T, k;
  const int32_t* sorted_rows;
  const uint16_t* a_src;
  uint16_t* h_out;
  float* y_out;           // down, fp32 rows (NULL when y16 is used)
  uint16_t* y16;          // down, fp16 rows already multiplied by their entry's gate
  const float* row_gate;  // LDS: gate of each of the tile's rows (y16 only)
  const int32_t* row_exp; // LDS: row exponent a of each of the tile's rows (x' = x 2^a; NULL: 0)
  uint32_t a_bytes;       // bytes of a_src, code and scale bytes of this expert
  uint32_t code_bytes, scale_bytes;
};

// MAXNMI = 32-row fragments per wave (tile height 32 MAXNMI: 32, 64 or 128
// rows); NMI <= MAXNMI the fragments this tile's rows need.  As holds three LDS
// buffers of the A tile.  128-row tiles run with the transposed accumulator
// (TR, see mfma_op).
// HALF (3-bit 32-row tiles): each wave takes one 32-column B fragment instead of
// two -- 16 gate + 16 up columns (gate/up) or 32 output columns (down) -- so a
// launch has twice the blocks, each with half the work and fewer registers
// (three blocks per compute unit instead of two).
template <bool GATEUP, int NMI, int MAXNMI, int DEPTH, bool Q3, bool HALF = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const GemmTile& t, uint16_t* As) {
  static_assert(!HALF || (MAXNMI == 1 && Q3), "half-width tiles: 32 rows, 3-bit");
  typedef typename std::conditional<Q3, typename std::conditional<HALF, BRegsH3, BRegs3>::type, BRegs>::type BRegs;
  constexpr bool TR = MAXNMI == 4;
  constexpr int BMX = 32 * MAXNMI;          // tile rows
  constexpr int NV = BMX / 32;              // 16-byte A chunks per thread and step
  constexpr int ABUF = BMX * A_STRIDE;      // halves per LDS buffer
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = GATEUP ? g.H : g.I;
  const int nch = K / GBK;

  // A staging: a step's tile is BMX rows x 8 chunks of 16 bytes; chunk
  // q * 256 + tid (row 32 q + tid / 8, chunk tid % 8) is this thread's q-th, so
  // every load instruction of a wave covers eight whole 128-byte row segments.
  // Rows past the tile's rows load its first row (no lane-divergent branch
  // around the loads; LDS rows past NMI * 32 are never read).
  const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(g.a_src, g.a_bytes);
  uint32_t a_voff[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int rr = 32 * q + (tid >> 3);
    const int pa = t.m0 + (rr < t.rows ? rr : 0);
    uint32_t arow;
    if (GATEUP) {
      const int r = g.sorted_rows[pa];
      const int Tk = g.T * g.k;
      arow = (uint32_t)(r < Tk ? r / g.k : r - Tk);
    } else {
      arow = (uint32_t)pa;
    }
    a_voff[q] = (arow * (uint32_t)K + (uint32_t)(tid & 7) * 8u) * 2u;
  }
  const int a_off = (tid >> 3) * A_STRIDE + (tid & 7) * 8;

  // B columns of this lane.  Gate/up with TR: lane m of the wave's 32 loads the
  // column whose pair-order position is m (position 2 j <- column j, 2 j + 1 <-
  // column 8 + j inside each 16-group), so accumulator rows come out in pair
  // order and h is stored as it is laid out.
  int n0, n1;
  if (HALF) {
    // lane m < 16 of each half-wave: gate column j; lane m + 16: up column j
    const int m = lane & 31;
    n0 = GATEUP ? (m < 16 ? 0 : g.I) + t.n * 64 + wv * 16 + (m & 15) : t.n * 128 + wv * 32 + m;
    n1 = n0;
  } else if (GATEUP) {
    const int m = lane & 31, j = m & 15;
    n0 = t.n * 128 + wv * 32 + (TR ? ((m & 16) | ((j & 1) ? 8 + (j >> 1) : (j >> 1))) : m);
    n1 = g.I + n0;
  } else {
    n0 = t.n * GCOLS + wv * 64 + (lane & 31);
    n1 = n0 + 32;
  }
  const BCol B0 = b_column(g.codes, g.scales, n0, K, Q3 ? g.hi : nullptr);
  const BCol B1 = b_column(g.codes, g.scales, n1, K, Q3 ? g.hi : nullptr);
  // 2-bit codes and scales through buffer loads: per-lane byte offsets of
  // column n0 (16 code bytes per step; 8 scale bytes per 128 K, the layout of
  // b_column) and the wave-uniform distance to column n1
  const __amdgpu_buffer_rsrc_t c_rsrc = buffer_rsrc(g.codes, g.code_bytes);
  const __amdgpu_buffer_rsrc_t s_rsrc = buffer_rsrc(g.scales, g.scale_bytes);
  const uint32_t c_voff = (uint32_t)((((n0 >> 6) * (K / 64)) * 64 + (n0 & 63)) * 16);
  const uint32_t s_voff = (uint32_t)((((n0 >> 6) * (K / 128)) * 64 + (n0 & 63)) * 8);
  const uint32_t c_d1 = HALF ? 0u : __builtin_amdgcn_readfirstlane(
      (uint32_t)((((n1 >> 6) * (K / 64)) * 64 + (n1 & 63)) * 16) - c_voff);
  const uint32_t s_d1 = HALF ? 0u : __builtin_amdgcn_readfirstlane(
      (uint32_t)((((n1 >> 6) * (K / 128)) * 64 + (n1 & 63)) * 8) - s_voff);
  const int shift = (lane >> 5) * 8, hshift = (lane >> 5) * 4;
  const BConst bc = bconst();
  BConstHi bch;
  if constexpr (Q3) bch = bconst_hi();

  f16x_t acc[MAXNMI][2];
#pragma unroll
  for (int i = 0; i < MAXNMI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Loads past the last step re-load the last step (index clamped): every load
  // is unconditional, so the wait counts before each use stay exact.
  struct ARegs {
    u32x4 a[NV];
  };
  auto load_a = [&](int kc, ARegs& R) {
    kc = kc < nch ? kc : nch - 1;
#pragma unroll
    for (int q = 0; q < NV; ++q) R.a[q] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff[q], kc * 128, 0);
  };
  auto store_a = [&](const ARegs& R, int buf) {
#pragma unroll
    for (int q = 0; q < NV; ++q) *reinterpret_cast<u32x4*>(As + buf * ABUF + a_off + 32 * q * A_STRIDE) = R.a[q];
  };
  auto load_bc = [&](int kc, BRegs& R) {
    kc = kc < nch ? kc : nch - 1;
    if constexpr (HALF) {
      // one column: as load_b for B0
      R.c0 = B0.codes[(size_t)kc * 64];
      R.s0 = B0.scales[(size_t)(kc >> 1) * 128 + (kc & 1)];
      R.h0 = B0.hi[(size_t)kc * 64];
    } else if constexpr (Q3) {
      load_b(B0, B1, kc, R);
    } else {
      // codes: 1024 bytes per step; scales: blocks 2 kc, 2 kc + 1 at dword
      // (kc / 2) * 128 + kc % 2
      const int so = (kc >> 1) * 512 + (kc & 1) * 4;
      R.c0 = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, c_voff, kc * 1024, 0);
      R.s0 = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_voff, so, 0);
      R.c1 = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, c_voff, kc * 1024 + c_d1, 0);
      R.s1 = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_voff, so + s_d1, 0);
    }
  };

  auto compute = [&](const uint16_t* Ab, const BRegs& Bc) {
    if constexpr (HALF)
      wave_step_half3(Ab, Bc, shift, hshift, bc, bch, acc[0][0]);
    else
      wave_step<NMI, MAXNMI, Q3, TR>(Ab, Bc, shift, hshift, bc, bch, acc);
  };

  if constexpr (DEPTH == 2) {
    // Three register sets with static names (the loop is unrolled by three).
    // Step m computes from LDS buffer m % 3 and B set m % 3; it first writes A
    // of step m + 1 (set (m + 1) % 3, loaded two steps earlier) into LDS buffer
    // (m + 1) % 3, then issues the loads of A for step m + 3 and of B for step
    // m + 2.  The scheduling barrier keeps the loads at the top of the step.
    ARegs AX, AY, AZ;
    BRegs BX, BY, BZ;
    load_a(0, AX);
    load_bc(0, BX);
    load_a(1, AY);
    load_bc(1, BY);
    load_a(2, AZ);
    store_a(AX, 0);
    __syncthreads();
#define MOE_GEMM_STEP3(J, ACUR1, ANEW, BCUR, BNEW)                   \
  {                                                                  \
    store_a(ACUR1, (J + 1) % 3);                                     \
    load_a(kc + J + 3, ANEW);                                        \
    load_bc(kc + J + 2, BNEW);                                       \
    __builtin_amdgcn_sched_barrier(0);                               \
    pin_b(BCUR);                                                     \
    compute(As + J * ABUF, BCUR);                                    \
    __syncthreads();                                                 \
  }
    // whole groups of three steps with no branch inside (exact wait counts),
    // then the remaining zero, one or two steps
    int kc = 0;
    for (; kc + 3 <= nch; kc += 3) {
      MOE_GEMM_STEP3(0, AY, AX, BX, BZ)
      MOE_GEMM_STEP3(1, AZ, AY, BY, BX)
      MOE_GEMM_STEP3(2, AX, AZ, BZ, BY)
    }
    if (kc < nch) MOE_GEMM_STEP3(0, AY, AX, BX, BZ)
    if (kc + 1 < nch) MOE_GEMM_STEP3(1, AZ, AY, BY, BX)
#undef MOE_GEMM_STEP3
  } else {
  // Register rings of R = DEPTH + 1 sets for A and B and three LDS buffers for
  // A.  Step m computes from LDS buffer m % 3 and B set m % R; it first writes
  // A of step m + 1 (set (m + 1) % R, loaded DEPTH steps earlier) into LDS
  // buffer (m + 1) % 3, then issues the loads of A for step m + DEPTH + 1 and
  // of B for step m + DEPTH.  The loop is unrolled by lcm(R, 3) so every ring
  // index is a compile-time constant (the sets stay in registers); the
  // scheduling barrier keeps the loads at the top of the step.
  constexpr int R = DEPTH + 1;
  constexpr int U = R % 3 == 0 ? R : 3 * R;
  ARegs Ar[R];
  BRegs Br[R];
#pragma unroll
  for (int i = 0; i <= DEPTH; ++i) load_a(i, Ar[i]);
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_bc(i, Br[i]);
  store_a(Ar[0], 0);
  __syncthreads();
#define MOE_GEMM_STEP(J)                                                       \
  {                                                                            \
    store_a(Ar[(J + 1) % R], (J + 1) % 3);                                     \
    load_a(kc + J + DEPTH + 1, Ar[J % R]);                                     \
    load_bc(kc + J + DEPTH, Br[(J + DEPTH) % R]);                              \
    __builtin_amdgcn_sched_barrier(0);                                         \
    pin_b(Br[J % R]);                                                          \
    compute(As + (J % 3) * ABUF, Br[J % R]);                                   \
    __syncthreads();                                                           \
  }
  // whole groups of U steps with no branch inside (exact wait counts), then
  // the remaining steps
  int kc = 0;
  for (; kc + U <= nch; kc += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) MOE_GEMM_STEP(j)
  }
#pragma unroll
  for (int j = 0; j < U - 1; ++j)
    if (kc + j < nch) MOE_GEMM_STEP(j)
#undef MOE_GEMM_STEP
  }

  if constexpr (TR) {
    // lane: token row 32 mi + l % 32; registers 4 q .. 4 q + 3: columns
    // 8 q + 4 (l / 32) + (0..3) of the wave's 32 (gate/up, pair-order
    // positions) or of each of its two 32-column halves f (down)
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int l32 = lane & 31, c4 = 4 * (lane >> 5);
    auto pack2 = [](float a, float b) {
      return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
    };
    if (GATEUP) {
      // h = SiLU(gate) * up in fp16, 8-byte stores
      const int hb = t.n * 128 + wv * 32 + c4;
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) {
        const int row = mi * 32 + l32;
        if (row < t.rows) {
          uint16_t* dst = g.h_out + (size_t)(t.m0 + row) * g.I + hb;
          const int ae = g.row_exp ? g.row_exp[row] : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) hv[j] = swiglu_scaled(acc[mi][0][4 * q + j], acc[mi][1][4 * q + j], ae);
            *reinterpret_cast<u2v*>(dst + 8 * q) = u2v{pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
          }
        }
      }
    } else if (g.y16) {
      // gate-scaled fp16 rows through LDS (the A buffers are free after the K
      // loop's last barrier): each wave writes its own 64 rows x 64 columns
      // region in 8-byte pieces, reads it back as 16-byte row chunks and
      // stores whole 128-byte row segments; two rounds of 64 rows.  Rows of 68
      // halves keep both LDS passes free of bank conflicts.
      constexpr int RS = 68;
      static_assert(4 * 64 * RS <= 3 * ABUF, "epilogue staging exceeds the A buffers");
      uint16_t* W = As + wv * (64 * RS);
      const int cb = t.n * GCOLS + wv * 64;
#pragma unroll
      for (int hr = 0; hr < (NMI + 1) / 2; ++hr) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int mi = 2 * hr + mm;
          if (mi < NMI) {
            const float gt = g.row_gate[mi * 32 + l32];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f16x_t& c = acc[mi][f];
                *reinterpret_cast<u2v*>(W + (mm * 32 + l32) * RS + f * 32 + 8 * q + c4) =
                    u2v{pack2(gt * c[4 * q], gt * c[4 * q + 1]), pack2(gt * c[4 * q + 2], gt * c[4 * q + 3])};
              }
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = i * 64 + lane, rl = idx >> 3, ch = idx & 7, row = hr * 64 + rl;
          const u2v lo = *reinterpret_cast<const u2v*>(W + rl * RS + ch * 8);
          const u2v hi = *reinterpret_cast<const u2v*>(W + rl * RS + ch * 8 + 4);
          if (row < t.rows)
            *reinterpret_cast<u32x4*>(g.y16 + (size_t)(t.m0 + row) * g.H + cb + ch * 8) = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    } else {
      // fp32 rows, 16-byte stores
      const int cb = t.n * GCOLS + wv * 64 + c4;
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) {
        const int row = mi * 32 + l32;
        if (row < t.rows) {
          float* dst = g.y_out + (size_t)(t.m0 + row) * g.H + cb;
          const int ue = g.row_exp ? -2 * g.row_exp[row] : 0;   // y = y' 4^-a
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<f4v*>(dst + 32 * f + 8 * q) =
                  f4v{ldexpf(acc[mi][f][4 * q], ue), ldexpf(acc[mi][f][4 * q + 1], ue),
                      ldexpf(acc[mi][f][4 * q + 2], ue), ldexpf(acc[mi][f][4 * q + 3], ue)};
        }
      }
    }
    return;
  }
  if (HALF && GATEUP) {
    // lanes m < 16 of each half-wave hold gate column j, lanes m + 16 the up
    // column j of the same rows: one exchange, then the gate lanes store h
    const int m = lane & 31;
    const int col = t.n * 64 + wv * 16 + (m & 15);
    const int pcol = (col & ~15) + pair_pos(col & 15);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float mine = acc[0][0][r];
      const float other = __shfl_xor(mine, 16, 64);
      const int row = acc_row(r, lane);
      if (m < 16 && row < t.rows) {
        const float hv = swiglu_scaled(mine, other, g.row_exp ? g.row_exp[row] : 0);
        g.h_out[(size_t)(t.m0 + row) * g.I + pcol] = __builtin_bit_cast(uint16_t, (_Float16)hv);
      }
    }
    return;
  }
  if (HALF) {
    // down: fp32 column n0 of each row (y16 is not used with 3-bit weights)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(r, lane);
      if (row < t.rows)
        g.y_out[(size_t)(t.m0 + row) * g.H + n0] = ldexpf(acc[0][0][r], g.row_exp ? -2 * g.row_exp[row] : 0);
    }
    return;
  }
  if (GATEUP) {
    // h = SiLU(gate) * up, fp16, stored at the pair-order position of its column
    const int col = t.n * 128 + wv * 32 + (lane & 31);
    const int pcol = (col & ~15) + pair_pos(col & 15);
#pragma unroll
    for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mi * 32 + acc_row(r, lane);
        if (row < t.rows) {
          const float hv = swiglu_scaled(acc[mi][0][r], acc[mi][1][r], g.row_exp ? g.row_exp[row] : 0);
          g.h_out[(size_t)(t.m0 + row) * g.I + pcol] = __builtin_bit_cast(uint16_t, (_Float16)hv);
        }
      }
  } else if (g.y16) {
#pragma unroll
    for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + acc_row(r, lane);
          if (row < t.rows)
            g.y16[(size_t)(t.m0 + row) * g.H + (f ? n1 : n0)] =
                __builtin_bit_cast(uint16_t, (_Float16)(g.row_gate[row] * acc[mi][f][r]));
        }
  } else {
#pragma unroll
    for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + acc_row(r, lane);
          if (row < t.rows)
            g.y_out[(size_t)(t.m0 + row) * g.H + (f ? n1 : n0)] =
                ldexpf(acc[mi][f][r], g.row_exp ? -2 * g.row_exp[row] : 0);
        }
  }
}

struct GemmKArgs {
  MatRef routed, shared;
  int H, I, E, T, k;
  const int32_t* tiles;
  const int32_t* n_tiles;
  const int32_t* sorted_rows;
  const uint16_t* a_src;
  uint16_t* h_out;
  float* y_out;
  const float* gates;
  uint16_t* y16;
  const int32_t* slot_map;   // expert-cache mode: pool slot of routed group g, or -1 (a miss)
  const int32_t* xexp;       // row exponent of each token (x' = x 2^a), or NULL (a = 0)
  MxTables mx;               // fp8-piece tables of the fp8 x fp4 tiles
};

static constexpr int kMxTileMaxI = 768;
#ifndef MOE_MX_DEPTH
#define MOE_MX_DEPTH 2
#endif
static constexpr int kMxDepth = MOE_MX_DEPTH;   // 256-column code chunks in flight per wave (gate/up)
bool mx_tiles_ok(int H, int I) {
  return H % 256 == 0 && H <= kMxTileMaxH && (I == 512 || I == 640 || I == 768);
}

// An fp8 x fp4 tile (mx_group.h) on the block's 4 waves: the rows' tables into
// LDS, then each wave's columns.
template <bool GATEUP>
__device__ __forceinline__ void gemm_tile_mx(const GemmKArgs& a, const GemmTile& t, const MatRef& M, size_t eidx,
                                             uint8_t* lds) {
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(M.codes + eidx * M.code_stride, (uint32_t)M.code_stride);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(M.scales + eidx * M.scale_stride, (uint32_t)(M.scale_stride * 2));
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // source rows of the tables: the token of each entry (x), or the sorted
  // position itself (h); rows past the tile repeat its last row (never read)
  int src[kMxTileRows];
#pragma unroll
  for (int j = 0; j < kMxTileRows; ++j) {
    const int p = t.m0 + (j < t.rows ? j : t.rows - 1);
    if (GATEUP) {
      const int r = a.sorted_rows[p], Tk = a.T * a.k;
      src[j] = r < Tk ? r / a.k : r - Tk;
    } else {
      src[j] = p;
    }
  }
  // each wave issues its first code loads, then the block stages the tables
  if (GATEUP) {
    auto stage = [&] {
      mx_stage<kMxTileMaxH>(lds, a.mx.x_data, a.mx.x_exps, a.H, t.rows, src);
      __syncthreads();
    };
    mx_tile_gateup<kMxDepth>(lds, t.rows, a.H, a.I, t.n * 128 + 32 * wv, rc, rs, t.m0, a.mx.h_data, a.mx.h_exps,
                             stage);
  } else {
    auto stage = [&] {
      mx_stage<kMxTileMaxI>(lds, a.mx.h_data, a.mx.h_exps, a.I, t.rows, src);
      __syncthreads();
    };
    const int o0 = t.n * GCOLS + 64 * wv;
    if (a.I == 512)
      mx_tile_down<2, 0>(lds, t.rows, a.H, o0, rc, rs, t.m0, a.y_out, stage);
    else if (a.I == 640)
      mx_tile_down<2, 1>(lds, t.rows, a.H, o0, rc, rs, t.m0, a.y_out, stage);
    else
      mx_tile_down<3, 0>(lds, t.rows, a.H, o0, rc, rs, t.m0, a.y_out, stage);
  }
}

// One kernel per projection, tile height and format: MAXNMI = 4 (128-row
// tiles, 2-bit, for prompt chunks) or 1 (32-row tiles, for verify batches of
// many sequences, whose experts have a few to a few dozen rows; 2-bit, or 3-bit
// with half-width tiles).
// In expert-cache mode a tile whose group has no slot computes nothing: the
// down projection writes zero rows, so the combine adds nothing for it.
// The 2-bit 32-row kernels also run the fp8 x fp4 tiles of small groups (MX);
// their LDS holds either the three A buffers or the staged tables.
template <bool GATEUP, int MAXNMI, bool Q3, bool HALF = false>
__global__ __launch_bounds__(256, (MAXNMI == 4 || (Q3 && !HALF)) ? 2 : 3) void k_gemm_q2(GemmKArgs a) {
  constexpr int BCOLS = HALF ? 128 : GCOLS;   // output columns of a down block
  constexpr bool MX = MAXNMI == 1 && !Q3;
  constexpr int AS_BYTES = 3 * 32 * MAXNMI * A_STRIDE * 2;
  constexpr int MX_BYTES = MX ? mx_stage_bytes(GATEUP ? kMxTileMaxH : kMxTileMaxI) : 0;
  __shared__ __attribute__((aligned(16))) uint8_t lds[AS_BYTES > MX_BYTES ? AS_BYTES : MX_BYTES];
  uint16_t* As = reinterpret_cast<uint16_t*>(lds);
  __shared__ float row_gate[32 * MAXNMI];
  __shared__ int32_t row_exp[32 * MAXNMI];
  GemmTile t;
  if (!load_tile(a.tiles, a.n_tiles, t)) return;
  const bool sh = t.g == a.E;
  int slot = t.g;
  if (a.slot_map && !sh) {
    slot = a.slot_map[t.g];
    if (slot < 0) {
      if (!GATEUP) {
        for (int i = threadIdx.x; i < t.rows * BCOLS; i += blockDim.x)
          a.y_out[(size_t)(t.m0 + i / BCOLS) * a.H + t.n * BCOLS + i % BCOLS] = 0.0f;
      }
      return;
    }
  }
  if constexpr (MX) {
    if (t.mx) {
      gemm_tile_mx<GATEUP>(a, t, sh ? a.shared : a.routed, sh ? 0 : (size_t)slot, lds);
      return;
    }
  }
  if (!GATEUP && a.y16) {
    // gate of every row of the tile (1 for the shared expert), read in the
    // epilogue after the K loop's barriers
    for (int i = threadIdx.x; i < t.rows; i += blockDim.x) {
      const int r = a.sorted_rows[t.m0 + i];
      row_gate[i] = r < a.T * a.k ? a.gates[r] : 1.0f;
    }
  }
  if (a.xexp) {
    // exponent of every row's token, read in the epilogue after the K loop's barriers
    for (int i = threadIdx.x; i < t.rows; i += blockDim.x) {
      const int r = a.sorted_rows[t.m0 + i];
      row_exp[i] = a.xexp[r < a.T * a.k ? r / a.k : r - a.T * a.k];
    }
  }
  const MatRef& M = sh ? a.shared : a.routed;
  const size_t eidx = sh ? 0 : (size_t)slot;
  GemmArgs g;
  g.codes = M.codes + eidx * M.code_stride;
  g.scales = M.scales + eidx * M.scale_stride;
  g.hi = Q3 ? M.hi + eidx * M.hi_stride : nullptr;
  g.H = a.H;
  g.I = a.I;
  g.T = a.T;
  g.k = a.k;
  g.sorted_rows = a.sorted_rows;
  g.a_src = a.a_src;
  g.h_out = a.h_out;
  g.y_out = a.y_out;
  g.y16 = a.y16;
  g.row_gate = row_gate;
  g.row_exp = a.xexp ? row_exp : nullptr;
  // byte sizes of the buffer resources (the host checks that they fit 31 bits)
  g.a_bytes = GATEUP ? (uint32_t)a.T * (uint32_t)a.H * 2u : (uint32_t)(a.T * a.k + a.T) * (uint32_t)a.I * 2u;
  g.code_bytes = (uint32_t)M.code_stride;
  g.scale_bytes = (uint32_t)(M.scale_stride * 2);
  // prefetch depth: two steps for 128-row tiles (register budget), five for
  // 32-row tiles (few rows: latency, not the matrix cores, sets the pace),
  // three with the 3-bit high-bit planes
  constexpr int D = MAXNMI == 4 ? 2 : (Q3 ? 3 : 5);
  const int nmi = __builtin_amdgcn_readfirstlane((t.rows + 31) >> 5);
  if (MAXNMI == 1 || nmi == 1) {
    gemm_tile<GATEUP, 1, MAXNMI, D, Q3, HALF>(g, t, As);
  } else if (MAXNMI == 2 || nmi == 2) {
    gemm_tile<GATEUP, (MAXNMI >= 2 ? 2 : 1), MAXNMI, D, Q3>(g, t, As);
  } else if (nmi == 3) {
    gemm_tile<GATEUP, (MAXNMI >= 4 ? 3 : 1), MAXNMI, D, Q3>(g, t, As);
  } else {
    gemm_tile<GATEUP, MAXNMI, MAXNMI, D, Q3>(g, t, As);
  }
}

template <int MAXNMI, bool Q3, bool HALF = false>
static hipError_t launch_gemm_q2_t(GemvKind kind, GemmKArgs a, int max_tiles, void* out, hipStream_t s) {
  if (kind == GemvKind::GateUp) {
    a.h_out = (uint16_t*)out;
    MOE_LAUNCH((k_gemm_q2<true, MAXNMI, Q3, HALF>), dim3(max_tiles, a.I / (HALF ? 64 : 128)), dim3(256), 0, s, a);
  } else {
    a.y_out = a.y16 ? nullptr : (float*)out;
    MOE_LAUNCH((k_gemm_q2<false, MAXNMI, Q3, HALF>), dim3(max_tiles, a.H / (HALF ? 128 : GCOLS)), dim3(256), 0, s,
               a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_q2(GemvKind kind, const MatRef& routed, const MatRef& shared, int H, int I, int E,
                          const int32_t* tiles, const int32_t* n_tiles, int max_tiles, const int32_t* sorted_rows,
                          int T, int k, const uint16_t* a_f16, void* out, hipStream_t s, const float* gates,
                          uint16_t* y16, int tile_rows, bool q3, const int32_t* slot_map, const int32_t* xexp,
                          const MxTables* mx) {
  if (max_tiles <= 0) return hipSuccess;
  // fp8 x fp4 tiles: 2-bit 32-row tiles writing fp32 rows
  if (mx && (q3 || tile_rows != 32 || y16 || !mx_tiles_ok(H, I) || !mx->x_data || !mx->h_data))
    return hipErrorInvalidValue;
  // the kernels address activations and one expert's weights with 32-bit
  // buffer offsets
  const uint64_t a_bytes = kind == GemvKind::GateUp ? (uint64_t)T * H * 2 : (uint64_t)T * (k + 1) * I * 2;
  if (a_bytes > 0x7FFFFFFFu || routed.code_stride > 0x7FFFFFFFu || shared.code_stride > 0x7FFFFFFFu)
    return hipErrorInvalidValue;
  GemmKArgs a = {};
  a.routed = routed;
  a.shared = shared;
  a.H = H;
  a.I = I;
  a.E = E;
  a.T = T;
  a.k = k;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.sorted_rows = sorted_rows;
  a.a_src = a_f16;
  a.gates = gates;
  a.y16 = y16;
  a.slot_map = slot_map;
  a.xexp = xexp;
  if (mx) a.mx = *mx;
  if (q3) {
    // 3-bit weights run on 32-row tiles only (the 128-row kernel's registers
    // have no room for the high-bit planes), half-width; y16 is not used with them
    if (tile_rows != 32 || y16) return hipErrorInvalidValue;
    return launch_gemm_q2_t<1, true, true>(kind, a, max_tiles, out, s);
  }
  if (tile_rows == 32) return launch_gemm_q2_t<1, false>(kind, a, max_tiles, out, s);
  return launch_gemm_q2_t<GBM / 32, false>(kind, a, max_tiles, out, s);
}

// ---------------------------------------------------------------------------
// Router GEMM (bf16 MFMA): logits[t, e] = x_t . Wr[e] + b[e] for 128 x 128 tiles.
// Both operands are bf16 in natural column order; products are exact in fp32.
//
// A prompt chunk has few tiles (8,192 tokens x 512 experts is one tile per
// compute unit), so one block per compute unit must hide its own latencies.
// The block has 8 waves, two per SIMD: waves 0-3 take the first half of K and
// waves 4-7 the second (H is a multiple of 128, so each half is a whole number
// of 64-column steps), each half with its own two LDS buffers of the A and B
// tiles, so that one half's LDS traffic and barriers overlap the other's MFMAs.
// At the end the second half's accumulators go through LDS and the first half
// adds them (first half + second half) and stores.  Each wave computes 64
// tokens x 64 experts.
// A half keeps RDEPTH K-steps of both operands in flight in registers.  Step m:
// write step m + 1 (loaded RDEPTH - 1 steps earlier) into the other LDS buffer,
// issue the loads of step m + RDEPTH into the register set just freed, then
// 4 x 4 MFMAs per wave from LDS (fragments read one 16-K sub-step ahead).  The
// loop is unrolled by RDEPTH so that every register set has a static name.
// Tile (m, n) is block n + 4 m of a linear order whose neighbours share one
// XCD, so the expert tiles of a token tile read its rows from one L2.
// ---------------------------------------------------------------------------
static constexpr int RDEPTH = 4;

__device__ __forceinline__ b8_t lds_frag_b(const uint16_t* base, int row, int k) {
  return *reinterpret_cast<const b8_t*>(base + row * LDS_STRIDE + k);
}

static constexpr int KH = 2;   // K halves

__global__ __launch_bounds__(256 * KH, 1) void k_router_mfma(const uint16_t* __restrict__ x, int T,
                                                             const uint16_t* __restrict__ wr,
                                                             const float* __restrict__ bias, int E, int H,
                                                             float* __restrict__ logits) {
  constexpr int TILE = BM * LDS_STRIDE;   // halves per LDS tile buffer
  // [half][buffer] A tiles, then [half][buffer] B tiles; the second half's
  // accumulators reuse the space at the end (4 x 2 x 2 x 16 x 64 floats)
  __shared__ __attribute__((aligned(16))) uint16_t lds[KH * 4 * TILE > 32768 ? KH * 4 * TILE : 32768];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = wv >> 2, wq = wv & 3, t = tid & 255;
  const int ntn = (E + BN - 1) / BN, ntm = (T + BM - 1) / BM;
  const int n_valid = ntm * ntn;
  const int lin = blockIdx.x;
  if (lin >= n_valid) return;
  const int per = (n_valid + 7) / 8, xcd = lin & 7, slot = lin >> 3;
  const int full = n_valid - 8 * (per - 1);
  const int id = xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
  const int m0 = (id / ntn) * BM, n0 = (id % ntn) * BN;
  uint16_t* As = lds + (size_t)half * 2 * TILE;
  uint16_t* Bs = lds + (size_t)(KH + half) * 2 * TILE;
  // staging: chunk q * 256 + t of a step is row 32 q + t / 8, 16-byte chunk
  // t % 8 (whole 128-byte row segments per load instruction); rows past T or
  // E load the last row and are never stored
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
  const __amdgpu_buffer_rsrc_t wrr = buffer_rsrc(wr, (uint32_t)E * (uint32_t)H * 2u);
  const int nch = H / BK / KH;           // K steps of this half
  const int kbase = half * nch * 128;    // byte offset of the half's K range in a row
  uint32_t xo[4], wo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = 32 * q + (t >> 3);
    xo[q] = ((uint32_t)min(m0 + rr, T - 1) * (uint32_t)H + (uint32_t)(t & 7) * 8u) * 2u + kbase;
    wo[q] = ((uint32_t)min(n0 + rr, E - 1) * (uint32_t)H + (uint32_t)(t & 7) * 8u) * 2u + kbase;
  }
  const int st_off = (t >> 3) * LDS_STRIDE + (t & 7) * 8;
  struct Stage {
    u32x4 a[4], b[4];
  };
  auto load = [&](int kc, Stage& S) {
    kc = kc < nch ? kc : nch - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      S.a[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo[q], kc * 128, 0);
      S.b[q] = __builtin_amdgcn_raw_buffer_load_b128(wrr, wo[q], kc * 128, 0);
    }
  };
  auto store = [&](const Stage& S, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4*>(&As[buf * TILE + st_off + 32 * q * LDS_STRIDE]) = S.a[q];
      *reinterpret_cast<u32x4*>(&Bs[buf * TILE + st_off + 32 * q * LDS_STRIDE]) = S.b[q];
    }
  };
  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int a0 = (wq >> 1) * 64, b0 = (wq & 1) * 64;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  auto compute = [&](int buf) {
    const uint16_t* Ab = As + buf * TILE;
    const uint16_t* Bb = Bs + buf * TILE;
    b8_t fa[2][2], fb[2][2];
    auto frags = [&](int k, int u) {
      fa[u][0] = lds_frag_b(Ab, a0 + r32, 16 * k + kh);
      fa[u][1] = lds_frag_b(Ab, a0 + 32 + r32, 16 * k + kh);
      fb[u][0] = lds_frag_b(Bb, b0 + r32, 16 * k + kh);
      fb[u][1] = lds_frag_b(Bb, b0 + 32 + r32, 16 * k + kh);
    };
    frags(0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k + 1 < 4) frags(k + 1, (k + 1) & 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k & 1][i], fb[k & 1][j], acc[i][j], 0, 0, 0);
    }
  };
  Stage S[RDEPTH];
#pragma unroll
  for (int i = 0; i < RDEPTH; ++i) load(i, S[i]);
  store(S[0], 0);
  __syncthreads();
  // step kc + J uses LDS buffer J % 2 and, for its successor, register set (J + 1) % RDEPTH
  int kc = 0;
  for (; kc + RDEPTH <= nch; kc += RDEPTH) {
#pragma unroll
    for (int J = 0; J < RDEPTH; ++J) {
      store(S[(J + 1) % RDEPTH], (kc + J + 1) & 1);
      load(kc + J + RDEPTH, S[J]);
      compute((kc + J) & 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int J = 0; J < RDEPTH - 1; ++J) {
    if (kc + J < nch) {
      store(S[(J + 1) % RDEPTH], (kc + J + 1) & 1);
      compute((kc + J) & 1);
      __syncthreads();
    }
  }
  {
    // every wave is past its last LDS read (the loop's last barrier): the
    // second half's accumulators go to LDS, the first half adds them
    float* red = reinterpret_cast<float*>(lds);   // [wq][i][j][r][lane]
    if (half == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((((wq * 2 + i) * 2 + j) * 16) + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((((wq * 2 + i) * 2 + j) * 16) + r) * 64 + lane];
  }
  // The bias is added before any store, and the stores take no branch (an
  // element outside [T) x [E) gets an offset past the buffer's end, which the
  // store drops): a store behind a branch that needs a bias load made the
  // compiler wait for every store in flight before it.
  float bv[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) bv[ni] = bias ? bias[min(n0 + b0 + 32 * ni + r32, E - 1)] : 0.0f;
  const __amdgpu_buffer_rsrc_t lr = buffer_rsrc(logits, (uint32_t)T * (uint32_t)E * 4u);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + a0 + 32 * mi + acc_row(r, lane);
        const int col = n0 + b0 + 32 * ni + r32;
        const uint32_t off = row < T && col < E ? ((uint32_t)row * (uint32_t)E + (uint32_t)col) * 4u : 0xFFFFFFF0u;
        const float v = acc[mi][ni][r] + bv[ni];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), lr, off, 0, 0);
      }
}

hipError_t launch_router_mfma(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s) {
  if ((uint64_t)T * H * 2 > 0x7FFFFFFFu || (uint64_t)E * H * 2 > 0x7FFFFFFFu || (uint64_t)T * E * 4 > 0x7FFFFFFFu)
    return hipErrorInvalidValue;
  if (H % (BK * KH)) return hipErrorInvalidValue;
  const int tiles = ((T + BM - 1) / BM) * ((E + BN - 1) / BN);
  MOE_LAUNCH(k_router_mfma, dim3(tiles), dim3(256 * KH), 0, s, x, T, wr, bias, E, H, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan: split the groups of a permutation between the MFMA GEMM (groups with at
// least min_rows entries, cut into tile_rows-row tiles) and the GEMV work items (the
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
                                               int items_per, int tile_rows, int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ n_tiles, int32_t* __restrict__ items,
                                               int32_t* __restrict__ n_items) {
  const int G = E + 1;
  const int g = threadIdx.x;
  const int start = g < G ? offsets[g] : 0;
  const int cnt = g < G ? offsets[g + 1] - start : 0;
  const bool big = cnt >= min_rows;
  const int nt = big ? (cnt + tile_rows - 1) / tile_rows : 0;
  const int ni = big ? 0 : (cnt + items_per - 1) / items_per;
  int tot_t = 0, tot_i = 0;
  const int pt = plan_scan_1024(nt, &tot_t);
  const int pi = plan_scan_1024(ni, &tot_i);
  for (int i = 0; i < nt; ++i) {
    tiles[3 * (pt + i)] = g;
    tiles[3 * (pt + i) + 1] = start + i * tile_rows;
    tiles[3 * (pt + i) + 2] = min(tile_rows, cnt - i * tile_rows);
  }
  for (int i = 0; i < ni; ++i) {
    items[3 * (pi + i)] = g;
    items[3 * (pi + i) + 1] = start + i * items_per;
    items[3 * (pi + i) + 2] = min(items_per, cnt - i * items_per);
  }
  if (g == 0) {
    n_tiles[0] = tot_t;
    n_tiles[1] = tot_t;   // all fp16 tiles
    *n_items = tot_i;
  }
}

hipError_t launch_plan(const int32_t* offsets, int E, int min_rows, int items_per, int32_t* tiles,
                       int32_t* n_tiles, int32_t* items, int32_t* n_items, hipStream_t s, int tile_rows) {
  MOE_LAUNCH(k_plan, dim3(1), dim3(1024), 0, s, offsets, E, min_rows, items_per, tile_rows > 0 ? tile_rows : GBM,
             tiles, n_tiles, items, n_items);
  return hipGetLastError();
}

int gemm_tile_rows() { return GBM; }
bool gemm_shape_ok(int H, int I) { return H % GCOLS == 0 && I % 128 == 0; }

}  // namespace moe

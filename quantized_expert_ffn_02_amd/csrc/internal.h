// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Every kernel launch goes through MOE_LAUNCH.  Inside a timed section (the
// C-ABI timing hook) the first launch carries the pending start event and
// every launch the stop event; hipExtLaunchKernel has the runtime stamp them
// from the kernel's own execution, so the elapsed time is kernel time, not
// kernel time plus the stream's dispatch gap.  Not thread-safe: the hook is a
// single-threaded measurement aid.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                              \
  do {                                                                                                  \
    ::moe::LaunchEvents& ev_ = ::moe::launch_events();                                                  \
    hipEvent_t start_ = ev_.start;                                                                      \
    ev_.start = nullptr;                                                                                \
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start_, ev_.stop, 0u, __VA_ARGS__);        \
  } while (0)

// One weight matrix of a bank: [n_experts] x [N rows x K cols].
struct MatRef {
  const uint8_t* codes = nullptr;     // Q2 codes / Q3 lo plane / bf16 values (as bytes)
  const uint8_t* hi = nullptr;        // Q3 hi plane
  const uint16_t* scales = nullptr;   // fp16 block scales
  size_t code_stride = 0;             // bytes per expert
  size_t hi_stride = 0;               // bytes per expert
  size_t scale_stride = 0;            // scales per expert
};

inline MatRef mat_w13(const moe_bank_t& b) {
  MatRef m;
  const size_t n = (size_t)2 * b.inter * b.hidden;
  m.codes = (const uint8_t*)b.w13;
  m.hi = (const uint8_t*)b.w13_hi;
  m.scales = b.w13_scale;
  m.code_stride = b.fmt == MOE_FMT_BF16 ? n * 2 : n / 4;
  m.hi_stride = n / 8;
  m.scale_stride = n / 32;
  return m;
}

inline MatRef mat_w2(const moe_bank_t& b) {
  MatRef m;
  const size_t n = (size_t)b.hidden * b.inter;
  m.codes = (const uint8_t*)b.w2;
  m.hi = (const uint8_t*)b.w2_hi;
  m.scales = b.w2_scale;
  m.code_stride = b.fmt == MOE_FMT_BF16 ? n * 2 : n / 4;
  m.hi_stride = n / 8;
  m.scale_stride = n / 32;
  return m;
}

// Groups of a permutation: group g < E is routed expert g, group E the shared
// expert.  The GEMV kernels walk "work items": (group, first sorted position,
// count <= items_per) triples covering every entry of every non-empty group,
// groups ascending, so a group with many tokens is spread over several blocks.
struct PermRef {
  const int32_t* offsets = nullptr;      // [E + 2]
  const int32_t* sorted_rows = nullptr;  // [n]
  const int32_t* items = nullptr;        // [max_items][3]: group, start, count
  const int32_t* n_items = nullptr;      // device scalar
  const int32_t* slot_map = nullptr;     // expert-cache mode: bank slot of routed expert g, or -1
  int32_t T = 0, k = 0, E = 0;
};

// Activation table of a quantized GEMV input (see k_prep_table): per row and
// 32-column block, ``sets`` x 16 packed bf16 pairs and one fp32 init value.
struct TableRef {
  const uint32_t* pairs = nullptr;   // [rows][K/32][sets][16]
  const float* init = nullptr;       // [rows][K/32]
  int sets = 1;
};

enum class GemvKind { GateUp, Down };

// Decode front end (router + activation table + top-k + small permutation), one launch.
struct SmallRouteArgs {
  const uint16_t* x;
  int T, E, H, k, with_shared, q3;
  const uint16_t* wr;
  const float* bias;
  float* logits;
  uint32_t* xpairs;    // activation table (NULL: not built)
  float* xinit;
  uint8_t* xmx_data = nullptr;   // fp8-piece activation table (mx.h; NULL: not built)
  uint8_t* xmx_exps = nullptr;
  // x before its RMSNorm: per-row partial sums of squares over 16-column runs
  // ([T][H / 16]) and eps; every use of x applies the norm (NULL: x is used as is)
  const float* norm_sq = nullptr;
  float norm_eps = 0.0f;
  int32_t* ids;
  float* gates;
  float* margin;       // may be NULL
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* row_to_sorted;
  int32_t* items;       // work items [n][3]
  int32_t* n_items;
  int items_per;        // entries per work item
};
// Largest T * k (+ T) the decode front end sorts in one block.
static constexpr int kSmallRouteMaxEntries = 1024;

// Decode-sized batches whose entries are addressed directly (decode_ffn.hip):
// no permutation, top-k inside the gate/up launch, combine inside the down
// launch.
static constexpr int kDecodeDirectMaxTokens = 16;
struct DecodeFfnArgs {
  MatRef r13, s13, r2, s2;
  int H = 0, I = 0, T = 0, k = 0, E = 0, with_shared = 0, q3 = 0;
  const float* logits = nullptr;      // [T][E] router logits
  int32_t* ids = nullptr;             // [T][k] written by the gate/up launch
  float* gates = nullptr;             // [T][k]
  float* margin = nullptr;            // [T] or NULL
  const uint32_t* xpairs = nullptr;   // activation table of x
  const float* xinit = nullptr;
  uint32_t* hpairs = nullptr;         // down projection's table of h, one row per entry
  float* hinit = nullptr;
  float* y = nullptr;                 // [entries][H] gate-scaled expert outputs
  const uint16_t* residual = nullptr; // [T][H] bf16 or NULL
  float* out = nullptr;               // [T][H]
  uint16_t* out_bf16 = nullptr;       // [T][H] or NULL
};
bool decode_direct_ok(int T, int k, int with_shared, int H, int I);

// The same decode FFN with 2-bit weights on the fp8 x fp4 matrix cores
// (decode_mx.hip, mx.h): activation tables of e4m3 pieces with block exponents.
struct MxFfnArgs {
  MatRef r13, s13, r2, s2;
  int H = 0, I = 0, T = 0, k = 0, E = 0, with_shared = 0;
  const float* logits = nullptr;      // [T][E] router logits
  int32_t* ids = nullptr;             // [T][k] written by the gate/up launch
  float* gates = nullptr;             // [T][k]
  float* margin = nullptr;            // [T] or NULL
  const uint8_t* xdata = nullptr;     // activation table of x, one row per token
  const uint8_t* xexps = nullptr;
  uint8_t* hdata = nullptr;           // table of h, one row per entry
  uint8_t* hexps = nullptr;
  float* y = nullptr;                 // [entries][H] gate-scaled expert outputs
};
bool decode_mx_ok(int H, int I, int q3);
hipError_t launch_decode_gateup_mx(const MxFfnArgs& a, hipStream_t s);
hipError_t launch_decode_down_mx(const MxFfnArgs& a, hipStream_t s);
// down projection and combine in one launch: a block per token and 64 output
// rows, a wave per entry (I in {512, 640, 768}, k + 1 <= 16 entries per token)
bool decode_down_combine_mx_ok(int I, int k, int with_shared);
// Byte ranges that a launch reads into the memory-side cache for a later launch (the
// next layer's weights that do not depend on its input: router rows, shared expert),
// in blocks after the launch's own.
struct Prefetch {
  static constexpr int kMax = 5;
  static constexpr int kPerThread = 2;   // 16-byte pieces per thread and range, all loads issued at once
  const void* ptr[kMax] = {};
  uint32_t bytes[kMax] = {};             // 0: unused range
  uint32_t max_bytes() const {
    uint32_t m = 0;
    for (int i = 0; i < kMax; ++i) m = bytes[i] > m ? bytes[i] : m;
    return m;
  }
};
// sq_out (may be NULL): partial sums of squares of the bf16 output per token and
// 64 rows ([T][H / 64]), the next layer's RMSNorm input; pf (may be NULL): ranges
// read by extra rows of blocks of the same launch, dispatched after its own
hipError_t launch_decode_down_combine_mx(const MxFfnArgs& a, const uint16_t* residual, float* out, uint16_t* out_bf16,
                                         float* sq_out, hipStream_t s, const Prefetch* pf = nullptr);
hipError_t launch_decode_gateup(const DecodeFfnArgs& a, hipStream_t s);
hipError_t launch_decode_down(const DecodeFfnArgs& a, hipStream_t s);
hipError_t launch_decode_combine(const DecodeFfnArgs& a, hipStream_t s);

// ---- launchers (return hipGetLastError()) ----
hipError_t launch_workspace_clear(void* ws, size_t bytes, hipStream_t s);
// RMSNorm that also writes the fp16 pair-order copy of its output (the grouped
// GEMM's activation layout, each row scaled by its exponent, written to xexp[T]),
// for H = 64 G, G <= 64
bool rmsnorm_f16_pairs_ok(int H);
hipError_t launch_rmsnorm_bf16_f16pairs(const uint16_t* x, int T, int H, float eps, uint16_t* out, uint16_t* f16p,
                                        int32_t* xexp, hipStream_t s);

hipError_t launch_router_gemv(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s);
hipError_t launch_router_mfma(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                              float* logits, hipStream_t s);
hipError_t launch_route_small(const SmallRouteArgs& a, hipStream_t s);
// router logits + activation table only (the first launch of launch_route_small)
hipError_t launch_route_front(const SmallRouteArgs& a, hipStream_t s);
// parts > 1: ``logits`` holds ``parts`` partial planes [T][E] to be added in
// plane order, then ``bias`` (launch_router_split with parts > 1).  With x set,
// the same launch also writes the grouped GEMMs' activation copy of x (as
// launch_x_to_f16_pairs: xf16 [T][H] and xexp [T]); topk_row_f16_ok(H).  With xmx_data
// set, extra blocks of the same launch write the fp8-piece table of xt (bf16 [T][H],
// H % 256 == 0; mx.h, 256-column form) for the fp8 x fp4 tiles of the grouped GEMM.
static constexpr int kRowF16MaxH = 3072;
bool topk_row_f16_ok(int H);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, int parts = 1, const float* bias = nullptr, const uint16_t* x = nullptr,
                       int H = 0, uint16_t* xf16 = nullptr, int32_t* xexp = nullptr, const uint16_t* xt = nullptr,
                       uint8_t* xmx_data = nullptr, uint8_t* xmx_exps = nullptr);

// permutation: counts/base are [n_chunks][E + 2] int32 scratch
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int with_shared, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* row_to_sorted, int32_t* counts, int32_t* base,
                          hipStream_t s);
int permute_chunks(int n_entries);
// permutation followed by the plan (launch_plan); batches of up to 16,384 entries
// in one single-block launch
// mx_rows > 0: every group of 1 .. mx_rows entries becomes ceil(entries / kMxTileRows)
// tiles of the fp8 x fp4 form (rows | kTileMx), listed after all the fp16 tiles;
// n_tiles[0] counts all tiles, n_tiles[1] the fp16 ones
hipError_t launch_permute_plan(const int32_t* ids, int T, int k, int E, int with_shared, int32_t* offsets,
                               int32_t* sorted_rows, int32_t* row_to_sorted, int32_t* counts, int32_t* base,
                               int min_rows, int items_per, int tile_rows, int32_t* tiles, int32_t* n_tiles,
                               int32_t* items, int32_t* n_items, hipStream_t s, int mx_rows = 0);
// work items of a permutation (see PermRef), from its offsets
hipError_t launch_items_from_offsets(const int32_t* offsets, int E, int items_per, int32_t* items,
                                     int32_t* n_items, hipStream_t s);

// activation tables
hipError_t launch_prep_table_bf16(const uint16_t* x, int rows, int K, bool q3, uint32_t* pairs, float* init,
                                  hipStream_t s);
hipError_t launch_prep_table_f32(const float* h, int rows, int K, bool q3, uint32_t* pairs, float* init,
                                 hipStream_t s);
hipError_t launch_bf16_rows_to_f32(const uint16_t* x, int rows, int K, float* out, hipStream_t s);

// dequant GEMV over the groups of a permutation
// GateUp: writes h = SiLU(gate) * up either as fp32 rows into ``out`` or, when
// down_pairs is set, directly as the down projection's activation table.
hipError_t launch_gemv_quant(GemvKind kind, int fmt, const MatRef& routed, const MatRef& shared, int N, int K,
                             int inter, const PermRef& perm, int max_groups, const TableRef& tab, float* out,
                             uint32_t* down_pairs, float* down_init, hipStream_t s);
hipError_t launch_gemv_dense(GemvKind kind, const MatRef& routed, const MatRef& shared, int N, int K, int inter,
                             const PermRef& perm, int max_groups, const float* in_rows, float* out,
                             hipStream_t s);

// MFMA path (gemm.hip)
// x' = x 2^a per row (a = -floor(log2 max|x_row|), written to xexp[T]) as fp16 in pair order
hipError_t launch_x_to_f16_pairs(const uint16_t* x, int T, int H, uint16_t* out, int32_t* xexp, hipStream_t s);
// The fp8-piece tables of the fp8 x fp4 tiles (2-bit, 32-row tiles): x [T] rows in the
// 256-column form (read), h [sorted position] rows in the mixed form (written by
// gate/up, read by down).
struct MxTables {
  const uint8_t* x_data = nullptr;
  const uint8_t* x_exps = nullptr;
  uint8_t* h_data = nullptr;
  uint8_t* h_exps = nullptr;
};
hipError_t launch_gemm_q2(GemvKind kind, const MatRef& routed, const MatRef& shared, int H, int I, int E,
                          const int32_t* tiles, const int32_t* n_tiles, int max_tiles, const int32_t* sorted_rows,
                          int T, int k, const uint16_t* a_f16, void* out, hipStream_t s, const float* gates = nullptr,
                          uint16_t* y16 = nullptr, int tile_rows = 128, bool q3 = false,
                          const int32_t* slot_map = nullptr, const int32_t* xexp = nullptr,
                          const MxTables* mx = nullptr);
// rows per tile of the grouped GEMM for batches beyond a decode step and below a prompt chunk
static constexpr int kSmallTileRows = 32;
// An expert group of at most kMxGroupRows entries on the 32-row 2-bit path runs on
// the block-scaled fp8 x fp4 matrix cores (the decode form, one product per row over
// codes loaded once) instead of dequantising the expert into fp16, in tiles of at
// most kMxTileRows rows; the plan marks them with kTileMx in the rows field.
// Shapes: mx_tiles_ok.  (Groups of 5 to 8 entries as two such tiles, each reading
// the expert's codes, were slower than one 32-row fp16 tile: 312 against 279 us for
// a 300-token verify batch.)
static constexpr int kMxTileRows = 4;
static constexpr int kMxGroupRows = 4;
static constexpr int kTileMx = 1 << 16;
static constexpr int kMxTileMaxH = 3072;
bool mx_tiles_ok(int H, int I);
// router of such batches (router_split.hip): 32 tokens x 64 experts per unit, K split over
// ``parts`` blocks (router_parts) and over the 4 waves of each; parts == 1 writes logits (with
// the bias), parts > 1 writes partial planes [parts][T][E] (without it) for launch_topk
int router_parts(int T, int E, int H);
hipError_t launch_router_split(const uint16_t* x, int T, const uint16_t* wr, const float* bias, int E, int H,
                               float* out, int parts, hipStream_t s);
// out[t] = 4^-a_t (sum over the token's entries of the gate-scaled fp16 rows y16,
// rank order, then the shared expert) (+ residual), fp32, optional bf16 copy;
// a_t = xexp[t] is the row exponent the rows were computed in (xexp NULL: 0)
hipError_t launch_combine16(const uint16_t* y16, const int32_t* row_to_sorted, int T, int k, int H, int with_shared,
                            const uint16_t* residual, float* out, uint16_t* out_bf16, const int32_t* xexp,
                            hipStream_t s);
hipError_t launch_plan(const int32_t* offsets, int E, int min_rows, int items_per, int32_t* tiles,
                       int32_t* n_tiles, int32_t* items, int32_t* n_items, hipStream_t s, int tile_rows = 0);
int gemm_tile_rows();
// shapes the grouped GEMM covers (column tiles of 128 gate/up and 256 down rows)
bool gemm_shape_ok(int H, int I);

// miss list of the expert-cache mode: entries r < T*k with slot_map[ids[r]] < 0, ascending
hipError_t launch_miss_list(const int32_t* ids, int Tk, const int32_t* slot_map, int32_t* miss_rows, int32_t* n_miss,
                            hipStream_t s);

// Up to kMax word ranges (src[i], words[i]; unused ranges have 0 words) copied back
// to back into dst.
struct PackWords {
  static constexpr int kMax = 5;
  const uint32_t* src[kMax] = {};
  uint32_t words[kMax] = {};
};
hipError_t launch_pack_words(const PackWords& p, uint32_t* dst, hipStream_t s);

// The combine (as launch_combine, out may be NULL, out_bf16 required) followed by
// the RMSNorm of its bf16 result into xn (and, if f16p, the scaled fp16 pair-order
// copy and its row exponents xexp), bit for bit as launch_rmsnorm_bf16_f16pairs on
// out_bf16.  combine_norm_ok(H).
bool combine_norm_ok(int H);
hipError_t launch_combine_norm(const float* y_sorted, const int32_t* row_to_sorted, const float* gates, int T, int k,
                               int H, int with_shared, const uint16_t* residual, float* out, uint16_t* out_bf16,
                               float eps, uint16_t* xn, uint16_t* f16p, int32_t* xexp, hipStream_t s);

// out[i] += y[i], i < n (both 16-byte aligned)
hipError_t launch_add_f32(float* out, const float* y, size_t n, hipStream_t s);

hipError_t launch_rmsnorm_bf16(const uint16_t* x, int T, int H, float eps, uint16_t* out, hipStream_t s);

hipError_t launch_combine(const float* y_sorted, const int32_t* row_to_sorted, const float* gates, int T, int k,
                          int H, int with_shared, const uint16_t* residual, float* out, uint16_t* out_bf16,
                          hipStream_t s);

}  // namespace moe

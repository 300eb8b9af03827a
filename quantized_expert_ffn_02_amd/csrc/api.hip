// C ABI of libmoe: host-side validation, workspace layout and kernel dispatch.
// Every argument check runs before the first HIP call, so invalid calls return
// an error code without touching the device.
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>

#include "internal.h"
#include "mx.h"

using namespace moe;

moe::LaunchEvents& moe::launch_events() {
  static LaunchEvents ev;
  return ev;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool fmt_ok(int f) { return f == MOE_FMT_BF16 || f == MOE_FMT_Q2 || f == MOE_FMT_Q3; }

int check_bank(const moe_bank_t& b, int n_experts_min, int H, int I) {
  if (!fmt_ok(b.fmt)) return MOE_EUNSUPPORTED;
  if (b.n_experts < n_experts_min || b.hidden != H || b.inter != I) return MOE_EINVAL;
  if (!b.w13 || !b.w2) return MOE_EINVAL;
  if (b.fmt != MOE_FMT_BF16 && (!b.w13_scale || !b.w2_scale)) return MOE_EINVAL;
  if (b.fmt == MOE_FMT_Q3 && (!b.w13_hi || !b.w2_hi)) return MOE_EINVAL;
  return MOE_OK;
}

int check_shape(const moe_layer_t* L) {
  if (!L) return MOE_EINVAL;
  if (L->hidden <= 0 || L->inter <= 0 || L->hidden % 128 || L->inter % 128) return MOE_EINVAL;
  if (L->n_experts < 1 || L->n_experts > 1023) return MOE_EINVAL;
  if (L->top_k < 1 || L->top_k > L->n_experts || L->top_k > 32) return MOE_EINVAL;
  return MOE_OK;
}

int check_layer(const moe_layer_t* L) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!L->w_router) return MOE_EINVAL;
  rc = check_bank(L->routed, L->n_experts, L->hidden, L->inter);
  if (rc) return rc;
  if (L->routed.n_experts != L->n_experts) return MOE_EINVAL;
  if (L->shared.fmt != MOE_FMT_NONE) {
    rc = check_bank(L->shared, 1, L->hidden, L->inter);
    if (rc) return rc;
    if (L->shared.fmt != L->routed.fmt) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

bool has_shared(const moe_layer_t* L) { return L->shared.fmt != MOE_FMT_NONE; }

// 1 <= T <= MOE_MAX_TOKENS (one prompt chunk at most)
bool tokens_ok(int32_t T) { return T >= 1 && T <= MOE_MAX_TOKENS; }

// Workspace layout of every call for a layer shape and up to T tokens.
struct Layout {
  size_t logits, rparts, ids, gates, margin;
  size_t counts, base, offsets, sorted_rows, row_to_sorted, items, n_items;
  size_t xtab_pairs, xtab_init, xf32, xf16, xexp, hf16, tiles, n_tiles;
  size_t h, htab_pairs, htab_init, y;
  size_t xmx_data, xmx_exps, hmx_data, hmx_exps;   // fp8-piece tables (mx.h)
  int64_t mx_tokens;                                // tokens those tables hold (entries: k + 1 each)
  size_t norm_sq;                                   // partial sums of squares of a stack layer's output
  size_t out_f32, xa, xb, xn;     // stack ping-pong buffers and the normalised layer input
  size_t miss_flag;
  size_t total;
};

Layout make_layout(const moe_layer_t* L, int64_t T) {
  const int64_t E = L->n_experts, k = L->top_k, H = L->hidden, I = L->inter;
  const int64_t n = T * k + T;   // room for the shared group
  const int64_t nc = permute_chunks((int)n);
  const int planes = L->routed.fmt == MOE_FMT_Q3 ? 2 : 1;
  const bool dense = L->routed.fmt == MOE_FMT_BF16;
  Layout o;
  size_t p = MOE_WS_CONTROL_BYTES;
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p = align_up(p + bytes);
    return at;
  };
  o.logits = take(T * E * 4);
  const int rp = router_parts((int)T, (int)E, (int)H);
  o.rparts = take(rp > 1 ? (size_t)rp * T * E * 4 : 0);   // K-split router partial planes
  o.ids = take(T * k * 4);
  o.gates = take(T * k * 4);
  o.margin = take(T * 4);
  o.counts = take(nc * (E + 2) * 4);
  o.base = take(nc * (E + 2) * 4);
  o.offsets = take((E + 2) * 4);
  o.sorted_rows = take(n * 4);
  o.row_to_sorted = take(n * 4);
  o.items = take(n * 3 * 4);
  o.n_items = take(4);
  o.xtab_pairs = take(dense ? 0 : T * (H / 32) * planes * 16 * 4);
  o.xtab_init = take(dense ? 0 : T * (H / 32) * 4);
  o.xf32 = take(dense ? T * H * 4 : 0);
  o.xf16 = take(dense ? 0 : T * H * 2);
  o.xexp = take(dense ? 0 : T * 4);   // row exponents of the fp16 copy
  o.hf16 = take(dense ? 0 : n * I * 2);
  o.tiles = take((n / kSmallTileRows + 2 * E + 3) * 3 * 4);   // GEMM tiles (128, 32 or 1 .. 4 rows)
  o.n_tiles = take(8);                                      // all tiles, fp16 tiles
  o.h = take(n * I * 4);
  o.htab_pairs = take(dense ? 0 : n * (I / 32) * planes * 2 * 16 * 4);
  o.htab_init = take(dense ? 0 : n * (I / 32) * 4);
  o.y = take(n * H * 4);
  // fp8-piece tables of the 2-bit decode batch (up to kDecodeDirectMaxTokens tokens),
  // and of the fp8 x fp4 tiles of a 2-bit batch on the 32-row GEMM path (any T below a
  // prompt chunk: x per token, h per entry)
  const bool q2 = L->routed.fmt == MOE_FMT_Q2;
  const bool mx = decode_mx_ok((int)H, (int)I, q2 ? 0 : 1) && !dense;
  const bool mxt = q2 && T > kDecodeDirectMaxTokens && T < 1024 && mx_tiles_ok((int)H, (int)I);
  const int64_t Tm = mxt ? T : mx ? (T < kDecodeDirectMaxTokens ? T : kDecodeDirectMaxTokens) : 0;
  const int64_t nm = Tm * k + Tm;
  o.mx_tokens = Tm;
  o.xmx_data = take(Tm * mx_data_bytes((int)H));
  o.xmx_exps = take(Tm * mx_exps_bytes((int)H));
  o.hmx_data = take(nm * mx_data_bytes((int)I));
  o.hmx_exps = take(nm * mx_exps_bytes((int)I));
  o.norm_sq = take(Tm * (H / 16) * 4);   // squares' sums per 16 output columns
  o.out_f32 = take(T * H * 4);
  o.xa = take(T * H * 2);
  o.xb = take(T * H * 2);
  o.xn = take(T * H * 2);
  o.miss_flag = take(T * k * 4);
  o.total = p;
  return o;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(void* ws, size_t ws_bytes, const Layout& lay) {
  if (!ws) return MOE_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_EWORKSPACE;
  if (ws_bytes < lay.total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// One-shot event pairs for moe_time_next_launch.
struct TimedLaunch {
  hipEvent_t start = nullptr, stop = nullptr;
};
TimedLaunch g_timed[MOE_KERNEL_COUNT];

// Runs ``launch`` with the pending events of ``kernel`` (if any) attached to
// its kernel launches (MOE_LAUNCH); if it launched nothing, both events are
// recorded on the stream so that they still hold a valid (empty) interval.
template <typename F>
hipError_t timed(int kernel, hipStream_t s, F&& launch) {
  TimedLaunch t = g_timed[kernel];
  if (!t.start) return launch();
  g_timed[kernel] = TimedLaunch();
  LaunchEvents& ev = launch_events();
  ev.start = t.start;
  ev.stop = t.stop;
  hipError_t e = launch();
  const bool none = ev.start != nullptr;
  ev = LaunchEvents();
  if (e != hipSuccess) return e;
  if (none) {
    e = hipEventRecord(t.start, s);
    if (e == hipSuccess) e = hipEventRecord(t.stop, s);
  }
  return e;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return MOE_EHIP; \
  } while (0)

// ---- steps shared by the public calls (arguments already validated) ----

int items_per_for(int T);
bool use_gemm_path(int n_entries);
int mfma_min_rows(int T);

// x_f16 (optional): when the top-k runs as its own launch (T > 16) it also writes
// the grouped GEMMs' scaled fp16 copy of x and its row exponents into the
// workspace; *x_f16 says whether it did.
// mx_table: the top-k launch of a verify batch also writes x's fp8-piece table (the
// fp8 x fp4 tiles of the 32-row GEMM path)
int do_route(const moe_layer_t* L, const uint16_t* x, int T, int32_t* ids, float* gates, float* margin, void* ws,
             const Layout& lay, hipStream_t s, bool* x_f16 = nullptr, bool mx_table = false) {
  const bool fuse = x_f16 && T > 16 && L->routed.fmt != MOE_FMT_BF16 && topk_row_f16_ok(L->hidden);
  const uint16_t* fx = fuse ? x : nullptr;
  uint16_t* fxf = fuse ? at<uint16_t>(ws, lay.xf16) : nullptr;
  int32_t* fxe = fuse ? at<int32_t>(ws, lay.xexp) : nullptr;
  if (x_f16) *x_f16 = fuse;
  float* logits = at<float>(ws, lay.logits);
  // split-K router partial planes (16 < T < 1024)
  const int parts = T > 16 && T < 1024 ? router_parts(T, L->n_experts, L->hidden) : 1;
  float* rparts = at<float>(ws, lay.rparts);
  MOE_TRY(timed(MOE_KERNEL_ROUTER, s, [&] {
    // prompt chunks: 128 x 128 MFMA tiles; verify batches: 32-token chunks with K
    // split over waves; a decode step: one wave per expert row
    if (T >= 1024) return launch_router_mfma(x, T, L->w_router, L->router_bias, L->n_experts, L->hidden, logits, s);
    if (T > 16)
      return launch_router_split(x, T, L->w_router, L->router_bias, L->n_experts, L->hidden,
                                 parts > 1 ? rparts : logits, parts, s);
    return launch_router_gemv(x, T, L->w_router, L->router_bias, L->n_experts, L->hidden, logits, s);
  }));
  uint8_t* tabd = mx_table ? at<uint8_t>(ws, lay.xmx_data) : nullptr;
  uint8_t* tabe = mx_table ? at<uint8_t>(ws, lay.xmx_exps) : nullptr;
  if (parts > 1)
    MOE_TRY(launch_topk(rparts, T, L->n_experts, L->top_k, ids, gates, margin, s, parts, L->router_bias, fx,
                        L->hidden, fxf, fxe, x, tabd, tabe));
  else
    MOE_TRY(launch_topk(logits, T, L->n_experts, L->top_k, ids, gates, margin, s, 1, nullptr, fx, L->hidden, fxf,
                        fxe, x, tabd, tabe));
  return MOE_OK;
}

// y16 (with gates): the prompt path, every group on the MFMA GEMM, whose down
// projection writes gate-scaled fp16 rows instead of fp32 y_sorted; no GEMV.
int do_expert_ffn(const moe_layer_t* L, const uint16_t* x, int T, const PermRef& perm, int n_entries,
                  float* y_sorted, void* ws, const Layout& lay, hipStream_t s, bool x_table_ready = false,
                  const int32_t* gemm_tiles = nullptr, const int32_t* n_gemm_tiles = nullptr,
                  const moe_bank_t* routed_override = nullptr, const float* gates = nullptr,
                  uint16_t* y16 = nullptr, bool x_f16_ready = false) {
  const moe_bank_t& rb = routed_override ? *routed_override : L->routed;
  const int H = L->hidden, I = L->inter, E = L->n_experts;
  // upper bound on GEMV work items: every entry, or, when the MFMA GEMM takes
  // the groups of min_rows or more entries, the items of the smaller groups
  int max_groups = n_entries;
  if (gemm_tiles) {
    const int mr = mfma_min_rows(T), ip = items_per_for(T);
    max_groups = std::min(n_entries, (E + 1) * ((mr - 1 + ip - 1) / ip));
  }
  const MatRef r13 = mat_w13(rb), r2 = mat_w2(rb);
  const MatRef s13 = has_shared(L) ? mat_w13(L->shared) : MatRef(), s2 = has_shared(L) ? mat_w2(L->shared) : MatRef();
  float* h = at<float>(ws, lay.h);
  if (rb.fmt == MOE_FMT_BF16) {
    float* xf = at<float>(ws, lay.xf32);
    MOE_TRY(launch_bf16_rows_to_f32(x, T, H, xf, s));
    MOE_TRY(launch_gemv_dense(GemvKind::GateUp, r13, s13, 2 * I, H, I, perm, max_groups, xf, h, s));
    MOE_TRY(launch_gemv_dense(GemvKind::Down, r2, s2, H, I, I, perm, max_groups, h, y_sorted, s));
    return MOE_OK;
  }
  const bool q3 = rb.fmt == MOE_FMT_Q3;
  TableRef xt;
  xt.pairs = at<uint32_t>(ws, lay.xtab_pairs);
  xt.init = at<float>(ws, lay.xtab_init);
  xt.sets = q3 ? 2 : 1;
  if (!x_table_ready && !y16)
    MOE_TRY(launch_prep_table_bf16(x, T, H, q3, const_cast<uint32_t*>(xt.pairs), const_cast<float*>(xt.init), s));
  TableRef ht;
  ht.pairs = at<uint32_t>(ws, lay.htab_pairs);
  ht.init = at<float>(ws, lay.htab_init);
  ht.sets = (q3 ? 2 : 1) * 2;
  // groups with many entries: MFMA grouped GEMM (2-bit banks)
  const bool gemm = gemm_tiles && !q3;
  const int max_tiles = gemm ? n_entries / gemm_tile_rows() + E + 2 : 0;
  uint16_t* hf = at<uint16_t>(ws, lay.hf16);
  int32_t* xexp = at<int32_t>(ws, lay.xexp);
  if (gemm) {
    uint16_t* xf = at<uint16_t>(ws, lay.xf16);
    if (!x_f16_ready) MOE_TRY(launch_x_to_f16_pairs(x, T, H, xf, xexp, s));
    MOE_TRY(timed(MOE_KERNEL_GATEUP_GEMM, s, [&] {
      return launch_gemm_q2(GemvKind::GateUp, r13, s13, H, I, E, gemm_tiles, n_gemm_tiles, max_tiles,
                            perm.sorted_rows, T, perm.k, xf, hf, s, nullptr, nullptr, gemm_tile_rows(), false,
                            nullptr, xexp);
    }));
  }
  if (!y16) {
    MOE_TRY(timed(MOE_KERNEL_GATEUP_GEMV, s, [&] {
      return launch_gemv_quant(GemvKind::GateUp, rb.fmt, r13, s13, 2 * I, H, I, perm, max_groups, xt, h,
                               const_cast<uint32_t*>(ht.pairs), const_cast<float*>(ht.init), s);
    }));
  }
  if (gemm) {
    MOE_TRY(timed(MOE_KERNEL_DOWN_GEMM, s, [&] {
      return launch_gemm_q2(GemvKind::Down, r2, s2, H, I, E, gemm_tiles, n_gemm_tiles, max_tiles,
                            perm.sorted_rows, T, perm.k, hf, y_sorted, s, gates, y16, gemm_tile_rows(), false,
                            nullptr, xexp);
    }));
  }
  if (y16) return MOE_OK;
  MOE_TRY(timed(MOE_KERNEL_DOWN_GEMV, s, [&] {
    return launch_gemv_quant(GemvKind::Down, rb.fmt, r2, s2, H, I, I, perm, max_groups, ht, y_sorted, nullptr,
                             nullptr, s);
  }));
  return MOE_OK;
}

// Entries per GEMV work item: one token per block for decode-sized batches
// (most parallel), four for larger batches.
int items_per_for(int T) { return T <= 16 ? 1 : 4; }

// Groups with at least this many entries go to the MFMA grouped GEMM (only for
// batches beyond the decode front end's size); smaller groups use the GEMV.
constexpr int kMfmaMinRows = 32;
// For a prompt-sized chunk every non-empty group goes to the GEMM.
int mfma_min_rows(int T) { return T >= 1024 ? 1 : kMfmaMinRows; }
bool use_gemm_path(int n_entries) { return n_entries > kSmallRouteMaxEntries; }

}  // namespace

extern "C" {

int moe_rmsnorm_bf16(const uint16_t* x, int32_t T, int32_t H, uint16_t* out, void* stream) {
  if (!x || !out || !tokens_ok(T) || H <= 0) return MOE_EINVAL;
  return hip_rc(launch_rmsnorm_bf16(x, T, H, MOE_RMS_EPS, out, (hipStream_t)stream));
}

int moe_time_next_launch(int32_t kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= MOE_KERNEL_COUNT) return MOE_EINVAL;
  if ((start_event == nullptr) != (stop_event == nullptr)) return MOE_EINVAL;
  g_timed[kernel].start = (hipEvent_t)start_event;
  g_timed[kernel].stop = (hipEvent_t)stop_event;
  return MOE_OK;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported format or shape";
    case MOE_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_EHIP: return "HIP launch error";
    case MOE_ESCRATCH: return "batch needs more than the built-in scratch of moe_layer_forward_noalloc";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_layer_t* L, int32_t T) {
  if (check_shape(L) || !tokens_ok(T)) return 0;
  if (!fmt_ok(L->routed.fmt)) return 0;
  return make_layout(L, T).total;
}

int moe_workspace_clear(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < MOE_WS_CONTROL_BYTES || reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_EWORKSPACE;
  return hip_rc(launch_workspace_clear(ws, MOE_WS_CONTROL_BYTES, (hipStream_t)stream));
}

int moe_route(const moe_layer_t* L, const uint16_t* x, int32_t T, int32_t* topk_ids, float* topk_gates,
              float* margin, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!L->w_router || !x || !topk_ids || !topk_gates || !tokens_ok(T)) return MOE_EINVAL;
  if (!fmt_ok(L->routed.fmt)) return MOE_EUNSUPPORTED;
  const Layout lay = make_layout(L, T);
  if ((rc = check_ws(ws, ws_bytes, lay))) return rc;
  return do_route(L, x, T, topk_ids, topk_gates, margin, ws, lay, (hipStream_t)stream);
}

int moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t with_shared, int32_t* offsets,
                int32_t* sorted_rows, int32_t* row_to_sorted, void* ws, size_t ws_bytes, void* stream) {
  if (!topk_ids || !offsets || !sorted_rows || !row_to_sorted) return MOE_EINVAL;
  if (!tokens_ok(T) || E < 1 || E > 1023 || k < 1 || k > E) return MOE_EINVAL;
  if ((int64_t)T * (k + 1) > (int64_t)1 << 30) return MOE_EINVAL;
  const int n = T * k + (with_shared ? T : 0);
  const int nc = permute_chunks(n);
  const size_t need = MOE_WS_CONTROL_BYTES + align_up((size_t)nc * (E + 2) * 4) * 2;
  if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign || ws_bytes < need) return MOE_EWORKSPACE;
  size_t p = MOE_WS_CONTROL_BYTES;
  int32_t* counts = at<int32_t>(ws, p);
  p += align_up((size_t)nc * (E + 2) * 4);
  int32_t* base = at<int32_t>(ws, p);
  return hip_rc(launch_permute(topk_ids, T, k, E, with_shared ? 1 : 0, offsets, sorted_rows, row_to_sorted, counts,
                               base, (hipStream_t)stream));
}

int moe_expert_ffn_q2(const moe_layer_t* L, const uint16_t* x, int32_t T, const int32_t* offsets,
                      const int32_t* sorted_rows, float* y_sorted, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !offsets || !sorted_rows || !y_sorted || !tokens_ok(T)) return MOE_EINVAL;
  const Layout lay = make_layout(L, T);
  if ((rc = check_ws(ws, ws_bytes, lay))) return rc;
  hipStream_t s = (hipStream_t)stream;
  PermRef perm;
  perm.offsets = offsets;
  perm.sorted_rows = sorted_rows;
  perm.items = at<int32_t>(ws, lay.items);
  perm.n_items = at<int32_t>(ws, lay.n_items);
  perm.T = T;
  perm.k = L->top_k;
  perm.E = L->n_experts;
  const int n = T * L->top_k + (has_shared(L) ? T : 0);
  const bool gemm = use_gemm_path(n) && L->routed.fmt == MOE_FMT_Q2 && gemm_shape_ok(L->hidden, L->inter);
  int32_t* tiles = at<int32_t>(ws, lay.tiles);
  int32_t* n_tiles = at<int32_t>(ws, lay.n_tiles);
  MOE_TRY(launch_plan(offsets, L->n_experts, gemm ? mfma_min_rows(T) : 0x7FFFFFFF, items_per_for(T), tiles, n_tiles,
                      const_cast<int32_t*>(perm.items), const_cast<int32_t*>(perm.n_items), s));
  return do_expert_ffn(L, x, T, perm, n, y_sorted, ws, lay, s, false, gemm ? tiles : nullptr,
                       gemm ? n_tiles : nullptr);
}

int moe_combine(const float* y_sorted, const int32_t* row_to_sorted, const float* topk_gates, int32_t T, int32_t k,
                int32_t H, int32_t with_shared, const uint16_t* residual, float* out, uint16_t* out_bf16,
                void* stream) {
  if (!y_sorted || !row_to_sorted || !topk_gates || !out) return MOE_EINVAL;
  if (!tokens_ok(T) || k < 1 || H <= 0 || H % 4) return MOE_EINVAL;
  return hip_rc(launch_combine(y_sorted, row_to_sorted, topk_gates, T, k, H, with_shared ? 1 : 0, residual, out,
                               out_bf16, (hipStream_t)stream));
}

// Batches beyond a decode step on the grouped MFMA GEMM with 32-row tiles
// (2-bit below a prompt chunk, 3-bit at any size): router, top-k, permutation,
// tile plan, x -> fp16 pair order, gate/up, down, combine.  In expert-cache
// mode ``routed`` is the slot pool and ``slot_map`` maps routed groups to pool
// slots (-1: a miss, whose rows contribute zero).
// The next stack layer's normalised input, written by this layer's combine.
struct NormNext {
  uint16_t* xn;     // bf16 RMSNorm of out_bf16
  uint16_t* f16p;   // its scaled fp16 pair-order copy (the next GEMM's input)
  int32_t* xexp;    // the copy's row exponents
  float eps;
};

// x_f16_ready: the workspace's fp16 pair-order copy of x is already written.
// after_route (optional) enqueues work that needs only the routing (ids, gates).
// norm_next (optional): the combine also writes the next layer's norm.
static int medium_path(const moe_layer_t* L, const moe_bank_t& routed, const int32_t* slot_map, const uint16_t* x,
                       int32_t T, const uint16_t* residual, float* out, uint16_t* out_bf16, int32_t* ids,
                       float* gates, float* margin, void* ws, const Layout& lay, hipStream_t s,
                       bool x_f16_ready = false, const std::function<int()>* after_route = nullptr,
                       const NormNext* norm_next = nullptr) {
  const int k = L->top_k, E = L->n_experts, H = L->hidden, I = L->inter;
  const int with_shared = has_shared(L) ? 1 : 0;
  const int n = T * k + (with_shared ? T : 0);
  int32_t* offsets = at<int32_t>(ws, lay.offsets);
  int32_t* srt = at<int32_t>(ws, lay.sorted_rows);
  int32_t* inv = at<int32_t>(ws, lay.row_to_sorted);
  bool xw = false;   // the top-k launch wrote the fp16 copy of x
  const bool q3 = routed.fmt == MOE_FMT_Q3;
  // groups of up to kMxTileRows entries on the fp8 x fp4 matrix cores (2-bit)
  const bool mxt = !q3 && T < 1024 && mx_tiles_ok(H, I) && lay.mx_tokens >= T;
  int rc = do_route(L, x, T, ids, gates, margin, ws, lay, s, x_f16_ready ? nullptr : &xw, mxt);
  if (rc) return rc;
  if (after_route && (rc = (*after_route)())) return rc;
  int32_t* chunks = at<int32_t>(ws, lay.tiles);
  int32_t* n_chunks = at<int32_t>(ws, lay.n_tiles);
  MOE_TRY(launch_permute_plan(ids, T, k, E, with_shared, offsets, srt, inv, at<int32_t>(ws, lay.counts),
                              at<int32_t>(ws, lay.base), 1, 1, kSmallTileRows, chunks, n_chunks,
                              at<int32_t>(ws, lay.items), at<int32_t>(ws, lay.n_items), s,
                              mxt ? kMxGroupRows : 0));
  // tiles: at most n / 32 + groups, and with fp8 x fp4 tiles one more for each group
  // of more than kMxTileRows entries (up to kMxGroupRows <= 2 kMxTileRows: two tiles)
  static_assert(kMxGroupRows <= 2 * kMxTileRows, "at most two fp8 x fp4 tiles per group");
  const int max_chunks = n / kSmallTileRows + std::min(E + 1, n) +
                         (mxt && kMxGroupRows > kMxTileRows ? std::min(n / (kMxTileRows + 1), E + 1) : 0) + 1;
  MxTables mxtab;
  mxtab.x_data = at<uint8_t>(ws, lay.xmx_data);
  mxtab.x_exps = at<uint8_t>(ws, lay.xmx_exps);
  mxtab.h_data = at<uint8_t>(ws, lay.hmx_data);
  mxtab.h_exps = at<uint8_t>(ws, lay.hmx_exps);
  const MatRef r13 = mat_w13(routed), r2 = mat_w2(routed);
  const MatRef s13 = with_shared ? mat_w13(L->shared) : MatRef(), s2 = with_shared ? mat_w2(L->shared) : MatRef();
  uint16_t* xf = at<uint16_t>(ws, lay.xf16);
  uint16_t* hf = at<uint16_t>(ws, lay.hf16);
  float* y = at<float>(ws, lay.y);
  // (a stack's normalised input comes with its fp16 copy and row exponents already written)
  int32_t* xexp = at<int32_t>(ws, lay.xexp);
  if (!x_f16_ready && !xw) MOE_TRY(launch_x_to_f16_pairs(x, T, H, xf, xexp, s));
  MOE_TRY(timed(MOE_KERNEL_GATEUP_GEMM, s, [&] {
    return launch_gemm_q2(GemvKind::GateUp, r13, s13, H, I, E, chunks, n_chunks, max_chunks, srt, T, k, xf, hf, s,
                          nullptr, nullptr, kSmallTileRows, q3, slot_map, xexp, mxt ? &mxtab : nullptr);
  }));
  MOE_TRY(timed(MOE_KERNEL_DOWN_GEMM, s, [&] {
    return launch_gemm_q2(GemvKind::Down, r2, s2, H, I, E, chunks, n_chunks, max_chunks, srt, T, k, hf, y, s,
                          nullptr, nullptr, kSmallTileRows, q3, slot_map, xexp, mxt ? &mxtab : nullptr);
  }));
  if (norm_next)
    MOE_TRY(launch_combine_norm(y, inv, gates, T, k, H, with_shared, residual, out, out_bf16, norm_next->eps,
                                norm_next->xn, norm_next->f16p, norm_next->xexp, s));
  else
    MOE_TRY(launch_combine(y, inv, gates, T, k, H, with_shared, residual, out, out_bf16, s));
  return MOE_OK;
}

// A batch between a decode step and a prompt chunk on the 32-row grouped GEMM.
static bool medium_path_taken(const moe_layer_t* L, int T) {
  return T > kDecodeDirectMaxTokens && gemm_shape_ok(L->hidden, L->inter) &&
         ((L->routed.fmt == MOE_FMT_Q2 && T < 1024) || L->routed.fmt == MOE_FMT_Q3);
}

// A layer whose decode batch takes the fp8 x fp4 path with the one-launch down
// and combine: its front end can apply the RMSNorm of its input, and its last
// launch can leave the partial sums of squares of its output.
static bool fused_norm_path(const moe_layer_t* L, int T) {
  const int k = L->top_k, with_shared = has_shared(L) ? 1 : 0;
  const int n = T * k + (with_shared ? T : 0);
  return L->routed.fmt == MOE_FMT_Q2 && T <= kDecodeDirectMaxTokens && n <= kSmallRouteMaxEntries &&
         decode_direct_ok(T, k, with_shared, L->hidden, L->inter) && decode_mx_ok(L->hidden, L->inter, 0) &&
         decode_down_combine_mx_ok(L->inter, k, with_shared);
}

// norm_sq_in: x is the layer input before its RMSNorm, with its partial sums of
// squares ([T][H / 16], per 16 columns); norm_sq_out: write those of out_bf16.
// Both only on the fused-norm decode path (fused_norm_path).
static int layer_forward_impl(const moe_layer_t* L, const uint16_t* x, int32_t T, const uint16_t* residual,
                              float* out, uint16_t* out_bf16, int32_t* topk_ids, float* topk_gates, float* margin,
                              void* ws, const Layout& lay, hipStream_t s, const float* norm_sq_in = nullptr,
                              float* norm_sq_out = nullptr, bool x_f16_ready = false,
                              const NormNext* norm_next = nullptr, const Prefetch* prefetch = nullptr) {
  if (norm_next && !medium_path_taken(L, T)) return MOE_EINVAL;   // only the 32-row GEMM path's combine writes it
  const int k = L->top_k, E = L->n_experts;
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, lay.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, lay.gates);
  const int with_shared = has_shared(L) ? 1 : 0;
  const int n = T * k + (with_shared ? T : 0);
  int32_t* offsets = at<int32_t>(ws, lay.offsets);
  int32_t* srt = at<int32_t>(ws, lay.sorted_rows);
  int32_t* inv = at<int32_t>(ws, lay.row_to_sorted);
  int32_t* items = at<int32_t>(ws, lay.items);
  int32_t* n_items = at<int32_t>(ws, lay.n_items);
  const bool quant = L->routed.fmt != MOE_FMT_BF16;
  bool x_table_ready = false, gemm = false, xw = false;   // xw: the top-k launch wrote the fp16 copy of x
  if (n <= kSmallRouteMaxEntries && quant && decode_direct_ok(T, k, with_shared, L->hidden, L->inter)) {
    // decode / MTP-verify batch, entries addressed directly: router front end,
    // gate/up with the top-k inside, down, combine
    SmallRouteArgs a;
    a.x = x;
    a.T = T;
    a.E = E;
    a.H = L->hidden;
    a.k = k;
    a.with_shared = with_shared;
    a.q3 = L->routed.fmt == MOE_FMT_Q3;
    a.wr = L->w_router;
    a.bias = L->router_bias;
    a.logits = at<float>(ws, lay.logits);
    if (decode_mx_ok(L->hidden, L->inter, a.q3)) {
      // 2-bit weights: the fp8 x fp4 matrix-core kernels
      a.xpairs = nullptr;
      a.xinit = nullptr;
      a.xmx_data = at<uint8_t>(ws, lay.xmx_data);
      a.xmx_exps = at<uint8_t>(ws, lay.xmx_exps);
      a.norm_sq = norm_sq_in;
      a.norm_eps = MOE_RMS_EPS;
      MOE_TRY(timed(MOE_KERNEL_ROUTER, s, [&] { return launch_route_front(a, s); }));
      MxFfnArgs m;
      m.r13 = mat_w13(L->routed);
      m.r2 = mat_w2(L->routed);
      if (with_shared) {
        m.s13 = mat_w13(L->shared);
        m.s2 = mat_w2(L->shared);
      }
      m.H = L->hidden;
      m.I = L->inter;
      m.T = T;
      m.k = k;
      m.E = E;
      m.with_shared = with_shared;
      m.logits = a.logits;
      m.ids = ids;
      m.gates = gates;
      m.margin = margin;
      m.xdata = a.xmx_data;
      m.xexps = a.xmx_exps;
      m.hdata = at<uint8_t>(ws, lay.hmx_data);
      m.hexps = at<uint8_t>(ws, lay.hmx_exps);
      m.y = at<float>(ws, lay.y);
      MOE_TRY(timed(MOE_KERNEL_GATEUP_GEMV, s, [&] { return launch_decode_gateup_mx(m, s); }));
      if (decode_down_combine_mx_ok(L->inter, k, with_shared)) {
        // down projection and combine in one launch (a block per token and 64 rows)
        MOE_TRY(timed(MOE_KERNEL_DOWN_GEMV, s,
                      [&] { return launch_decode_down_combine_mx(m, residual, out, out_bf16, norm_sq_out, s, prefetch); }));
        return MOE_OK;
      }
      MOE_TRY(timed(MOE_KERNEL_DOWN_GEMV, s, [&] { return launch_decode_down_mx(m, s); }));
      DecodeFfnArgs d;
      d.H = L->hidden;
      d.T = T;
      d.k = k;
      d.with_shared = with_shared;
      d.y = m.y;
      d.residual = residual;
      d.out = out;
      d.out_bf16 = out_bf16;
      MOE_TRY(launch_decode_combine(d, s));
      return MOE_OK;
    }
    a.xpairs = at<uint32_t>(ws, lay.xtab_pairs);
    a.xinit = at<float>(ws, lay.xtab_init);
    MOE_TRY(timed(MOE_KERNEL_ROUTER, s, [&] { return launch_route_front(a, s); }));
    DecodeFfnArgs d;
    d.r13 = mat_w13(L->routed);
    d.r2 = mat_w2(L->routed);
    if (with_shared) {
      d.s13 = mat_w13(L->shared);
      d.s2 = mat_w2(L->shared);
    }
    d.H = L->hidden;
    d.I = L->inter;
    d.T = T;
    d.k = k;
    d.E = E;
    d.with_shared = with_shared;
    d.q3 = a.q3;
    d.logits = a.logits;
    d.ids = ids;
    d.gates = gates;
    d.margin = margin;
    d.xpairs = a.xpairs;
    d.xinit = a.xinit;
    d.hpairs = at<uint32_t>(ws, lay.htab_pairs);
    d.hinit = at<float>(ws, lay.htab_init);
    d.y = at<float>(ws, lay.y);
    d.residual = residual;
    d.out = out;
    d.out_bf16 = out_bf16;
    MOE_TRY(timed(MOE_KERNEL_GATEUP_GEMV, s, [&] { return launch_decode_gateup(d, s); }));
    MOE_TRY(timed(MOE_KERNEL_DOWN_GEMV, s, [&] { return launch_decode_down(d, s); }));
    MOE_TRY(launch_decode_combine(d, s));
    return MOE_OK;
  }
  if (medium_path_taken(L, T))
    return medium_path(L, L->routed, nullptr, x, T, residual, out, out_bf16, ids, gates, margin, ws, lay, s,
                       x_f16_ready, nullptr, norm_next);
  if (n <= kSmallRouteMaxEntries) {
    // decode / MTP-verify batch: router, activation table, top-k and permutation in one launch
    SmallRouteArgs a;
    a.x = x;
    a.T = T;
    a.E = E;
    a.H = L->hidden;
    a.k = k;
    a.with_shared = with_shared;
    a.q3 = L->routed.fmt == MOE_FMT_Q3;
    a.wr = L->w_router;
    a.bias = L->router_bias;
    a.logits = at<float>(ws, lay.logits);
    a.xpairs = quant ? at<uint32_t>(ws, lay.xtab_pairs) : nullptr;
    a.xinit = quant ? at<float>(ws, lay.xtab_init) : nullptr;
    a.ids = ids;
    a.gates = gates;
    a.margin = margin;
    a.offsets = offsets;
    a.sorted_rows = srt;
    a.row_to_sorted = inv;
    a.items = items;
    a.n_items = n_items;
    a.items_per = items_per_for(T);
    MOE_TRY(timed(MOE_KERNEL_ROUTER, s, [&] { return launch_route_small(a, s); }));
    x_table_ready = quant;
  } else {
    gemm = L->routed.fmt == MOE_FMT_Q2 && gemm_shape_ok(L->hidden, L->inter);
    int rc = do_route(L, x, T, ids, gates, margin, ws, lay, s, gemm ? &xw : nullptr);
    if (rc) return rc;
    MOE_TRY(launch_permute_plan(ids, T, k, E, with_shared, offsets, srt, inv, at<int32_t>(ws, lay.counts),
                                at<int32_t>(ws, lay.base), gemm ? mfma_min_rows(T) : 0x7FFFFFFF, items_per_for(T),
                                gemm_tile_rows(), at<int32_t>(ws, lay.tiles), at<int32_t>(ws, lay.n_tiles), items,
                                n_items, s));
  }
  PermRef perm;
  perm.offsets = offsets;
  perm.sorted_rows = srt;
  perm.items = items;
  perm.n_items = n_items;
  perm.T = T;
  perm.k = k;
  perm.E = E;
  float* y = at<float>(ws, lay.y);
  // a prompt-sized chunk puts every group on the GEMM: gate-scaled fp16 rows
  uint16_t* y16 = gemm && mfma_min_rows(T) == 1 ? at<uint16_t>(ws, lay.y) : nullptr;
  int rc = do_expert_ffn(L, x, T, perm, n, y, ws, lay, s, x_table_ready, gemm ? at<int32_t>(ws, lay.tiles) : nullptr,
                         gemm ? at<int32_t>(ws, lay.n_tiles) : nullptr, nullptr, gates, y16, xw);
  if (rc) return rc;
  if (y16)
    MOE_TRY(launch_combine16(y16, inv, T, k, L->hidden, with_shared, residual, out, out_bf16,
                             at<int32_t>(ws, lay.xexp), s));
  else
    MOE_TRY(launch_combine(y, inv, gates, T, k, L->hidden, with_shared, residual, out, out_bf16, s));
  return MOE_OK;
}

int moe_layer_forward(const moe_layer_t* L, const uint16_t* x, int32_t T, const uint16_t* residual, float* out,
                      uint16_t* out_bf16, int32_t* topk_ids, float* topk_gates, float* margin, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !out || !tokens_ok(T)) return MOE_EINVAL;
  const Layout lay = make_layout(L, T);
  if ((rc = check_ws(ws, ws_bytes, lay))) return rc;
  return layer_forward_impl(L, x, T, residual, out, out_bf16, topk_ids, topk_gates, margin, ws, lay,
                            (hipStream_t)stream);
}

}  // extern "C"

// Workspace of moe_layer_forward_noalloc: one array per GPU in the library's code
// object, so using it needs no allocation.  Host code never passes the array's name
// to a kernel (in host code it is a stand-in, not a device address): it looks up
// each device's own address once with hipGetSymbolAddress and uses that.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch of the current device (looked up on the first call with it current).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const moe_layer_t* L, const uint16_t* x, int32_t T, const uint16_t* residual,
                              float* out, uint16_t* out_bf16, int32_t* topk_ids, float* topk_gates, float* margin,
                              void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !out || !tokens_ok(T)) return MOE_EINVAL;
  const Layout lay = make_layout(L, T);
  if (lay.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void* ws = nullptr;
  if ((rc = current_scratch(&ws))) return rc;
  return layer_forward_impl(L, x, T, residual, out, out_bf16, topk_ids, topk_gates, margin, ws, lay,
                            (hipStream_t)stream);
}

int moe_stack_forward(const moe_layer_t* layers, int32_t n_layers, const uint16_t* x0, int32_t T, uint16_t* x_out,
                      float* out_last, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 1 || !x0 || !x_out || !tokens_ok(T)) return MOE_EINVAL;
  int rc;
  size_t need = 0;
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_layer(&layers[l]))) return rc;
    if (layers[l].hidden != layers[0].hidden) return MOE_EINVAL;
    need = std::max(need, make_layout(&layers[l], T).total);
  }
  if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign || ws_bytes < need) return MOE_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* cur = x0;
  // On the fused-norm decode path a layer leaves the partial sums of squares of
  // its output, and the next layer's front end applies the RMSNorm as it loads
  // x (no separate norm launch); otherwise the norm runs on its own.
  bool have_sq = false;
  size_t sq_off = 0;
  // Between two layers of one shape on the 32-row GEMM path, the first one's
  // combine writes the second one's normalised input and its fp16 copy (same
  // workspace layout, so those regions are free by then); no norm launch.
  bool norm_done = false;
  auto same_shape = [](const moe_layer_t& a, const moe_layer_t& b) {
    return a.hidden == b.hidden && a.n_experts == b.n_experts && a.top_k == b.top_k && a.inter == b.inter &&
           a.routed.fmt == b.routed.fmt && a.shared.fmt == b.shared.fmt;
  };
  for (int l = 0; l < n_layers; ++l) {
    const Layout lay = make_layout(&layers[l], T);
    uint16_t* nxt = (l == n_layers - 1) ? x_out : at<uint16_t>(ws, (l % 2) ? lay.xb : lay.xa);
    float* of = (l == n_layers - 1 && out_last) ? out_last : at<float>(ws, lay.out_f32);
    const bool fused = fused_norm_path(&layers[l], T);
    const bool norm_in = have_sq && fused && lay.norm_sq == sq_off;
    const bool norm_out = fused && l + 1 < n_layers;
    float* sq = at<float>(ws, lay.norm_sq);
    const uint16_t* lin = cur;
    // on the 32-row GEMM path the norm also writes the GEMM's fp16 copy of its output
    const bool f16 = !norm_in && medium_path_taken(&layers[l], T) && layers[l].routed.fmt != MOE_FMT_BF16 &&
                     rmsnorm_f16_pairs_ok(layers[l].hidden);
    if (norm_done) {
      lin = at<uint16_t>(ws, lay.xn);
    } else if (!norm_in) {
      uint16_t* xn = at<uint16_t>(ws, lay.xn);
      if (f16)
        MOE_TRY(launch_rmsnorm_bf16_f16pairs(cur, T, layers[l].hidden, MOE_RMS_EPS, xn, at<uint16_t>(ws, lay.xf16),
                                             at<int32_t>(ws, lay.xexp), s));
      else
        MOE_TRY(launch_rmsnorm_bf16(cur, T, layers[l].hidden, MOE_RMS_EPS, xn, s));
      lin = xn;
    }
    NormNext nn;
    const NormNext* next = nullptr;
    if (f16 && l + 1 < n_layers && same_shape(layers[l], layers[l + 1]) && combine_norm_ok(layers[l].hidden)) {
      nn.xn = at<uint16_t>(ws, lay.xn);
      nn.f16p = at<uint16_t>(ws, lay.xf16);
      nn.xexp = at<int32_t>(ws, lay.xexp);
      nn.eps = MOE_RMS_EPS;
      next = &nn;
    }
    // on the fused-norm decode path the layer's last launch also reads the next
    // layer's router rows and shared expert into the memory-side cache
    Prefetch pf;
    if (fused && l + 1 < n_layers) {
      const moe_layer_t& Ln = layers[l + 1];
      pf.ptr[0] = Ln.w_router;
      pf.bytes[0] = (uint32_t)((size_t)Ln.n_experts * Ln.hidden * 2);
      if (has_shared(&Ln)) {
        const MatRef s13 = mat_w13(Ln.shared), s2 = mat_w2(Ln.shared);
        pf.ptr[1] = s13.codes;
        pf.bytes[1] = (uint32_t)s13.code_stride;
        pf.ptr[2] = s13.scales;
        pf.bytes[2] = (uint32_t)(s13.scale_stride * 2);
        pf.ptr[3] = s2.codes;
        pf.bytes[3] = (uint32_t)s2.code_stride;
        pf.ptr[4] = s2.scales;
        pf.bytes[4] = (uint32_t)(s2.scale_stride * 2);
      }
    }
    // a layer whose combine writes the next layer's normalised input leaves no fp32
    // output (only the last layer's is returned)
    rc = layer_forward_impl(&layers[l], lin, T, cur, next ? nullptr : of, nxt, nullptr, nullptr, nullptr, ws, lay, s,
                            norm_in ? sq : nullptr, norm_out ? sq : nullptr, f16, next, pf.max_bytes() ? &pf : nullptr);
    if (rc) return rc;
    norm_done = next != nullptr;
    have_sq = norm_out;
    sq_off = lay.norm_sq;
    cur = nxt;
  }
  return MOE_OK;
}

// Expert-cache layer.  The miss list is enqueued right after the routing, then
// after_route (optional: the tiered layer's copy of the routing to the host), then
// the cached experts, the shared expert and the combine.
static int cached_layer(const moe_layer_t* L, int32_t layer_idx, int32_t n_layers, const int32_t* slot_of,
                        const moe_bank_t* slot_pool, const uint16_t* x, int32_t T, float* out, int32_t* topk_ids,
                        float* topk_gates, int32_t* miss_rows, int32_t* n_miss, void* ws, size_t ws_bytes,
                        hipStream_t s, const std::function<int()>* after_route, const int32_t** ids_out = nullptr,
                        const float** gates_out = nullptr) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!L->w_router || !slot_of || !slot_pool || !x || !out || !miss_rows || !n_miss || !tokens_ok(T))
    return MOE_EINVAL;
  if (n_layers < 1 || layer_idx < 0 || layer_idx >= n_layers) return MOE_EINVAL;
  if ((rc = check_bank(*slot_pool, 1, L->hidden, L->inter))) return rc;
  if (slot_pool->fmt == MOE_FMT_BF16) return MOE_EUNSUPPORTED;
  if (L->shared.fmt != MOE_FMT_NONE) {
    if ((rc = check_bank(L->shared, 1, L->hidden, L->inter))) return rc;
    if (L->shared.fmt != slot_pool->fmt) return MOE_EUNSUPPORTED;
  }
  // the slot pool stands in for the routed bank (same format and expert shape)
  moe_layer_t Lc = *L;
  Lc.routed = *slot_pool;
  Lc.routed.n_experts = L->n_experts;
  const Layout lay = make_layout(&Lc, T);
  if ((rc = check_ws(ws, ws_bytes, lay))) return rc;
  const int k = L->top_k, E = L->n_experts;
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, lay.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, lay.gates);
  if (ids_out) *ids_out = ids;
  if (gates_out) *gates_out = gates;
  const int with_shared = has_shared(L) ? 1 : 0;
  const int n = T * k + (with_shared ? T : 0);
  int32_t* offsets = at<int32_t>(ws, lay.offsets);
  int32_t* srt = at<int32_t>(ws, lay.sorted_rows);
  int32_t* inv = at<int32_t>(ws, lay.row_to_sorted);
  int32_t* items = at<int32_t>(ws, lay.items);
  int32_t* n_items = at<int32_t>(ws, lay.n_items);
  const int32_t* slot_map = slot_of + (size_t)layer_idx * E;
  const std::function<int()> routed = [&]() -> int {
    MOE_TRY(launch_miss_list(ids, T * k, slot_map, miss_rows, n_miss, s));
    return after_route ? (*after_route)() : MOE_OK;
  };
  if (T > kDecodeDirectMaxTokens && gemm_shape_ok(L->hidden, L->inter))
    return medium_path(&Lc, *slot_pool, slot_map, x, T, nullptr, out, nullptr, ids, gates, nullptr, ws, lay, s,
                       false, &routed);
  bool x_table_ready = false;
  if (n <= kSmallRouteMaxEntries) {
    SmallRouteArgs a;
    a.x = x;
    a.T = T;
    a.E = E;
    a.H = L->hidden;
    a.k = k;
    a.with_shared = with_shared;
    a.q3 = slot_pool->fmt == MOE_FMT_Q3;
    a.wr = L->w_router;
    a.bias = L->router_bias;
    a.logits = at<float>(ws, lay.logits);
    a.xpairs = at<uint32_t>(ws, lay.xtab_pairs);
    a.xinit = at<float>(ws, lay.xtab_init);
    a.ids = ids;
    a.gates = gates;
    a.margin = nullptr;
    a.offsets = offsets;
    a.sorted_rows = srt;
    a.row_to_sorted = inv;
    a.items = items;
    a.n_items = n_items;
    a.items_per = items_per_for(T);
    MOE_TRY(timed(MOE_KERNEL_ROUTER, s, [&] { return launch_route_small(a, s); }));
    x_table_ready = true;
  } else {
    rc = do_route(L, x, T, ids, gates, nullptr, ws, lay, s);
    if (rc) return rc;
    MOE_TRY(launch_permute_plan(ids, T, k, E, with_shared, offsets, srt, inv, at<int32_t>(ws, lay.counts),
                                at<int32_t>(ws, lay.base), 0x7FFFFFFF, items_per_for(T), gemm_tile_rows(),
                                at<int32_t>(ws, lay.tiles), at<int32_t>(ws, lay.n_tiles), items, n_items, s));
  }
  if ((rc = routed())) return rc;
  PermRef perm;
  perm.offsets = offsets;
  perm.sorted_rows = srt;
  perm.items = items;
  perm.n_items = n_items;
  perm.slot_map = slot_map;
  perm.T = T;
  perm.k = k;
  perm.E = E;
  float* y = at<float>(ws, lay.y);
  rc = do_expert_ffn(&Lc, x, T, perm, n, y, ws, lay, s, x_table_ready);
  if (rc) return rc;
  MOE_TRY(launch_combine(y, inv, gates, T, k, L->hidden, with_shared, nullptr, out, nullptr, s));
  return MOE_OK;
}

int moe_layer_forward_cached(const moe_layer_t* L, int32_t layer_idx, int32_t n_layers, const int32_t* slot_of,
                             const moe_bank_t* slot_pool, const uint16_t* x, int32_t T, float* out,
                             int32_t* topk_ids, float* topk_gates, int32_t* miss_rows, int32_t* n_miss, void* ws,
                             size_t ws_bytes, void* stream) {
  return cached_layer(L, layer_idx, n_layers, slot_of, slot_pool, x, T, out, topk_ids, topk_gates, miss_rows, n_miss,
                      ws, ws_bytes, (hipStream_t)stream, nullptr);
}

// Host staging of the tiered layer: x, ids, gates, miss rows and their count back
// to back (4-byte aligned; one copy from the device), then the miss sum.
struct HostStage {
  size_t x, ids, gates, rows, n_rows, packed, y, total;
};

static HostStage host_stage(const moe_layer_t* L, int64_t T) {
  const int64_t k = L->top_k, H = L->hidden;
  HostStage h;
  h.x = 0;
  h.ids = h.x + T * H * 2;
  h.gates = h.ids + T * k * 4;
  h.rows = h.gates + T * k * 4;
  h.n_rows = h.rows + T * k * 4;
  h.packed = h.n_rows + 4;
  h.y = align_up(h.packed);
  h.total = h.y + T * H * 4;
  return h;
}

size_t moe_tiered_host_bytes(const moe_layer_t* L, int32_t T) {
  if (check_shape(L) || !tokens_ok(T)) return 0;
  return host_stage(L, T).total;
}

int moe_layer_forward_tiered(const moe_layer_t* L, int32_t layer_idx, int32_t n_layers, const int32_t* slot_of,
                             const moe_bank_t* slot_pool, const moe_bank_t* host_bank, const uint16_t* x, int32_t T,
                             float* out, int32_t* topk_ids, float* topk_gates, int32_t* miss_rows, int32_t* n_miss,
                             void* ws, size_t ws_bytes, void* host_ws, size_t host_ws_bytes, int32_t n_threads,
                             void* stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!host_bank || !host_ws || !tokens_ok(T) || n_threads < 0) return MOE_EINVAL;
  if ((uintptr_t)x & 3) return MOE_EINVAL;   // copied to the host as 4-byte words
  if (!slot_pool) return MOE_EINVAL;
  if ((rc = check_bank(*host_bank, L->n_experts, L->hidden, L->inter))) return rc;
  if (host_bank->fmt != slot_pool->fmt) return MOE_EUNSUPPORTED;
  if (host_bank->fmt == MOE_FMT_BF16) return MOE_EUNSUPPORTED;
  if (moe_cpu_isa() == 0) return MOE_EUNSUPPORTED;
  const HostStage hs = host_stage(L, T);
  if (host_ws_bytes < hs.total || ((uintptr_t)host_ws & (kAlign - 1))) return MOE_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, H = L->hidden;
  char* hb = (char*)host_ws;
  hipEvent_t routed_ev = nullptr;
  const int32_t* ids = nullptr;
  const float* gates = nullptr;
  // The workspace's expert-output area stages the packed routing (before the cached
  // experts write it) and later the miss sum (after the combine has read it); the
  // stream orders both.  It holds T(k+1)H floats, more than the packed bytes.
  moe_layer_t Lc = *L;
  Lc.routed = *slot_pool;
  Lc.routed.n_experts = L->n_experts;
  float* dy = at<float>(ws, make_layout(&Lc, T).y);
  // after the routing and the miss list: one copy of them (and x) to the host, then an
  // event the host waits on
  const std::function<int()> to_host = [&]() -> int {
    PackWords pw;
    pw.src[0] = (const uint32_t*)x;
    pw.words[0] = (uint32_t)((size_t)T * H / 2);
    pw.src[1] = (const uint32_t*)ids;
    pw.src[2] = (const uint32_t*)gates;
    pw.src[3] = (const uint32_t*)miss_rows;
    pw.words[1] = pw.words[2] = pw.words[3] = (uint32_t)(T * k);
    pw.src[4] = (const uint32_t*)n_miss;
    pw.words[4] = 1;
    MOE_TRY(launch_pack_words(pw, (uint32_t*)dy, s));
    MOE_TRY(hipMemcpyAsync(hb, dy, hs.packed, hipMemcpyDeviceToHost, s));
    MOE_TRY(hipEventCreateWithFlags(&routed_ev, hipEventDisableTiming));
    MOE_TRY(hipEventRecord(routed_ev, s));
    return MOE_OK;
  };
  rc = cached_layer(L, layer_idx, n_layers, slot_of, slot_pool, x, T, out, topk_ids, topk_gates, miss_rows, n_miss,
                    ws, ws_bytes, s, &to_host, &ids, &gates);
  if (rc) {
    if (routed_ev) (void)hipEventDestroy(routed_ev);
    return rc;
  }
  // the GPU runs the cached experts meanwhile
  const hipError_t werr = hipEventSynchronize(routed_ev);
  (void)hipEventDestroy(routed_ev);
  if (werr != hipSuccess) return MOE_EHIP;
  const int32_t nm = *(const int32_t*)(hb + hs.n_rows);
  if (nm <= 0) return MOE_OK;
  float* hy = (float*)(hb + hs.y);
  rc = moe_cpu_expert_ffn(host_bank, (const uint16_t*)(hb + hs.x), T, k, (const int32_t*)(hb + hs.ids),
                          (const float*)(hb + hs.gates), (const int32_t*)(hb + hs.rows), nm, hy, n_threads);
  if (rc) return rc;
  MOE_TRY(hipMemcpyAsync(dy, hy, (size_t)T * H * 4, hipMemcpyHostToDevice, s));
  MOE_TRY(launch_add_f32(out, dy, (size_t)T * H, s));
  return MOE_OK;
}

}  // extern "C"

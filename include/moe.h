/*
 * moe.h -- C ABI of libmoe: one sparse mixture-of-experts layer with 2-bit (and
 * 3-bit / bf16) block-quantized experts, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (pages cited by title and section):
 *   - route each token to the 10 largest of 512 router logits, plus one always-on
 *     shared expert ("Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU at
 *     Up to 94 Tokens/s", section "What it is"; "Strata: a 125B AI model on your
 *     gaming PC", model spec table, rows "Experts" and "Hidden dimension");
 *   - run every selected expert's FFN from quantized weights (the Q2_0 2-bit build
 *     of the first page's section "The numbers, measured by the author") and sum
 *     the results weighted by the gates;
 *   - compute only the experts resident in a GPU cache and list the others as
 *     misses (first page, section "How a 125B model fits in 12 GB");
 *   - take decode batches of 1 + 3 MTP draft tokens and prompt chunks of up to
 *     8,192 tokens ("Strata Runs a 125-Billion-Parameter Qwen Model on a 12 GB
 *     Gaming GPU at up to 93 Tokens per Second", speculative decoding and
 *     chunked prompt reading).
 * The pages leave the router function, gate normalisation, FFN type and weight
 * layout open.  This library's reading: softmax router, top-k by logit with ties
 * to the lower expert index, gates = softmax renormalised over the k selected,
 * SwiGLU experts (h = SiLU(W_gate x) * (W_up x), y = W_down h) without biases,
 * shared expert added with weight 1, fp32 layer output.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *     owned by the caller, except in the host miss tier (moe_cpu_expert_ffn and
 *     moe_layer_forward_tiered), which says which of its arguments live in host
 *     memory and is the one part that blocks and is not capturable; structs
 *     (moe_layer_t, moe_bank_t) live in host memory and are read during the call
 *     only.  bf16 / fp16 values travel as uint16_t
 *     bit patterns.  Row-major unless stated.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls enqueue kernels and
 *     return without synchronising; they allocate nothing and call no memset, so
 *     they can be captured into a HIP graph.
 *   - Errors: arguments are validated on the host before any launch; a failed
 *     check returns MOE_EINVAL / MOE_EUNSUPPORTED / MOE_EWORKSPACE and enqueues
 *     nothing.  A launch failure returns MOE_EHIP.  Nothing is thrown.
 *   - Workspace: ``ws`` is caller-owned device memory of at least
 *     moe_workspace_bytes() bytes, 256-byte aligned.  Its first
 *     MOE_WS_CONTROL_BYTES hold counters that must be zero before the first call
 *     (allocate it zero-filled, or call moe_workspace_clear once); every call
 *     leaves them zero again.  Calls that share a workspace must not overlap.
 *   - Results are deterministic: no floating-point atomics; every sum has a
 *     fixed order, so re-running a call gives bit-identical outputs.
 *   - Batch size: every call that takes a token count T accepts 1 <= T <=
 *     MOE_MAX_TOKENS, the largest prompt chunk the pages read in one pass (second
 *     page cited above, chunked prompt reading); a longer prompt is fed as several
 *     calls.  Outside that range the call returns MOE_EINVAL (moe_workspace_bytes
 *     and moe_tiered_host_bytes return 0).
 *
 * Weight layouts (this library's own definition; the pages give none).
 * A matrix W has N rows (outputs) and K columns (inputs), N % 64 == 0 and
 * K % 128 == 0, cut into tiles of 64 rows x 64 columns numbered
 * t = (n / 64) * (K / 64) + k / 64.
 *   MOE_FMT_Q2  code c in 0..3, weight = s * (c - 2), s = fp16 scale of the
 *               row's 32-column block.  Code byte t*1024 + (n%64)*16 + (k%64)/4,
 *               bits 2*(k%4)..+1.  Scale index ((n/64)*(K/128) + (k/32)/4)*256
 *               + (n%64)*4 + (k/32)%4.  1,536,000 bytes per 2560x640 expert.
 *   MOE_FMT_Q3  c = lo + 4*hi in 0..7, weight = s * (c - 4).  ``lo`` has the Q2
 *               code layout; ``hi`` holds 8 bytes per (tile, row) at byte
 *               t*512 + (n%64)*8: writing k%64 = 16*w + j (w 0..3, j 0..15), the
 *               bit is number 32*(w/2) + 8*(w%2) + (j%8) + 16*(j/8) of that
 *               little-endian 64-bit word.  Scales as Q2.
 *   MOE_FMT_BF16 element (n, k) at ((n/64)*(K/8) + k/8)*512 + (n%64)*8 + k%8.
 * Each expert has W13 = [2I x H] (rows 0..I-1 gate, I..2I-1 up) and
 * W2 = [H x I] (down); a bank stores its experts back to back, expert-major.
 * The router weight is plain row-major bf16 [E x H].
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer, non-positive size, k > E, bad shape */
  MOE_EUNSUPPORTED = -2,  /* format or shape this build has no kernel for */
  MOE_EWORKSPACE = -3,    /* workspace missing, misaligned or too small */
  MOE_EHIP = -4,          /* a HIP launch reported an error */
  MOE_ESCRATCH = -5       /* the batch needs more than the built-in scratch (moe_layer_forward_noalloc) */
};

enum { MOE_FMT_NONE = -1, MOE_FMT_BF16 = 0, MOE_FMT_Q2 = 1, MOE_FMT_Q3 = 2 };

/* Bytes at the start of every workspace reserved for zero-initialised counters. */
#define MOE_WS_CONTROL_BYTES 65536

/* Largest token count T of one call. */
#define MOE_MAX_TOKENS 8192

/* A bank of n_experts experts in one format (device pointers, caller-owned). */
typedef struct moe_bank {
  int32_t fmt;                /* MOE_FMT_*; MOE_FMT_NONE = no bank */
  int32_t n_experts;
  int32_t hidden;             /* H */
  int32_t inter;              /* I */
  const void* w13;            /* Q2 codes / Q3 lo plane / bf16 values, n_experts * [2I x H] */
  const void* w13_hi;         /* Q3 hi plane, else NULL */
  const uint16_t* w13_scale;  /* fp16 block scales (Q2/Q3), else NULL */
  const void* w2;             /* same for the down projection, n_experts * [H x I] */
  const void* w2_hi;
  const uint16_t* w2_scale;
} moe_bank_t;

/* One MoE layer. */
typedef struct moe_layer {
  int32_t hidden;             /* H, multiple of 128 */
  int32_t n_experts;          /* E routed experts, <= 1023 */
  int32_t top_k;              /* k, 1 <= k <= min(E, 32) */
  int32_t inter;              /* I, multiple of 128 */
  const uint16_t* w_router;   /* bf16 [E x H] row-major */
  const float* router_bias;   /* fp32 [E] added to the logits, or NULL */
  moe_bank_t routed;          /* n_experts == E */
  moe_bank_t shared;          /* n_experts == 1, or fmt == MOE_FMT_NONE for no shared expert */
} moe_layer_t;

/* Workspace bytes needed by every call below for a layer of this shape and up
 * to T tokens (including MOE_WS_CONTROL_BYTES).  Returns 0 for invalid shapes. */
size_t moe_workspace_bytes(const moe_layer_t* L, int32_t T);

/* Zero the workspace's control region with a kernel (no memset), on ``stream``. */
int moe_workspace_clear(void* ws, size_t ws_bytes, void* stream);

/* Router: logits l[t,e] = sum_h x[t,h] Wr[e,h] (+ b[e]) in fp32 from bf16
 * inputs; topk_ids[t, 0..k-1] = the k largest logits in descending order, ties to
 * the lower expert index; topk_gates[t,i] = exp(l_i - l_0) / sum_j exp(l_j - l_0)
 * over the selected (= the softmax over all E renormalised over the k);
 * margin[t] = l_(k) - l_(k+1) (the gap below the last selected logit; +inf if
 * k == E), so callers can flag near-ties.
 * x bf16 [T x H]; topk_ids int32 [T x k]; topk_gates fp32 [T x k]; margin fp32 [T] or NULL. */
int moe_route(const moe_layer_t* L, const uint16_t* x, int32_t T,
              int32_t* topk_ids, float* topk_gates, float* margin,
              void* ws, size_t ws_bytes, void* stream);

/* Permutation of the routed entries r = t*k + i (and, if with_shared, the shared
 * entries r = T*k + t, as group E) by expert: a stable counting sort.
 * offsets int32 [E + 2]: offsets[g] = first sorted position of group g,
 * offsets[E + 1] = total entries; sorted_rows int32 [n]: the entry at each sorted
 * position, ascending r inside a group; row_to_sorted int32 [n]: the inverse.
 * n = T*k (+ T).  Expert ids must lie in [0, E). */
int moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t with_shared,
                int32_t* offsets, int32_t* sorted_rows, int32_t* row_to_sorted,
                void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs over a permutation: for every sorted position p holding entry r of
 * group g (token t = r / k for r < T*k, t = r - T*k for the shared group E),
 * y_sorted[p] = W_down,g ( SiLU(W_gate,g x[t]) * (W_up,g x[t]) ), fp32 [n x H].
 * The routed bank serves groups 0..E-1, the shared bank group E.  The bank
 * format picks the kernel (2-bit, 3-bit or bf16); groups with few tokens use
 * the dequant-GEMV kernels, groups with many tokens the MFMA grouped GEMM. */
int moe_expert_ffn_q2(const moe_layer_t* L, const uint16_t* x, int32_t T,
                      const int32_t* offsets, const int32_t* sorted_rows, float* y_sorted,
                      void* ws, size_t ws_bytes, void* stream);

/* Gate-weighted combine in a fixed order:
 * out[t] = sum_{i=0..k-1} g[t,i] y_sorted[row_to_sorted[t*k+i]]
 *          (+ y_sorted[row_to_sorted[T*k+t]] if with_shared) (+ residual[t]);
 * out fp32 [T x H]; out_bf16 (optional) = out rounded to bf16, nearest-even. */
int moe_combine(const float* y_sorted, const int32_t* row_to_sorted, const float* topk_gates,
                int32_t T, int32_t k, int32_t H, int32_t with_shared, const uint16_t* residual,
                float* out, uint16_t* out_bf16, void* stream);

/* The whole layer: route, permute, expert FFNs, shared expert, combine, as one call.
 * out fp32 [T x H] = MoE(x) (+ residual); out_bf16, topk_ids, topk_gates, margin
 * optional (NULL = not returned). */
int moe_layer_forward(const moe_layer_t* L, const uint16_t* x, int32_t T, const uint16_t* residual,
                      float* out, uint16_t* out_bf16, int32_t* topk_ids, float* topk_gates,
                      float* margin, void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, kernels and results as moe_layer_forward; the
 * workspace is a built-in device array of MOE_NOALLOC_SCRATCH_BYTES, one per GPU,
 * held from the library's first call of this function on that GPU until the process
 * ends.  It covers every batch whose moe_workspace_bytes() fits (at H = 2,560,
 * I = 640, 512 experts, top-10 + shared: up to T = 128 tokens in the 2-bit and the
 * 3-bit format); larger batches return MOE_ESCRATCH before anything is enqueued.
 * The scratch of the CURRENT device is used, so ``stream`` must belong to it.  The
 * call allocates nothing (no hipMalloc, no library allocation); the scratch's address
 * is looked up once per device, on the first call made with that device current.
 * Every call on one GPU shares that GPU's scratch and leaves its last contents there
 * (no part of it has to start at zero): calls that overlap on one GPU race, so
 * serialise them (one stream, or events). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int moe_layer_forward_noalloc(const moe_layer_t* L, const uint16_t* x, int32_t T, const uint16_t* residual,
                              float* out, uint16_t* out_bf16, int32_t* topk_ids, float* topk_gates,
                              float* margin, void* stream);

/* Parameter-free RMSNorm of each bf16 row: out = bf16(x / sqrt(mean(x^2) + eps)),
 * rounded to nearest even, fp32 arithmetic; x, out bf16 [T x H] (may not overlap). */
#define MOE_RMS_EPS 1e-6f
int moe_rmsnorm_bf16(const uint16_t* x, int32_t T, int32_t H, uint16_t* out, void* stream);

/* A stack of n_layers layers joined by residual adds (48 layers in the model, first
 * page, section "What it is"), each layer reading the RMS-normalised stream:
 *   x_{l+1} = bf16(x_l + MoE_l(RMSNorm(x_l)))
 * (the pages do not describe the normalisation around the MoE block; without one
 * a residual chain of random-weight SwiGLU experts diverges).  x0 bf16 [T x H];
 * x_out bf16 [T x H] = x_{n_layers} (must not overlap x0); out_last (optional)
 * fp32 [T x H] = the last layer's fp32 x + MoE(RMSNorm(x)).  ``layers`` is a host
 * array of n_layers layer structs. */
int moe_stack_forward(const moe_layer_t* layers, int32_t n_layers, const uint16_t* x0, int32_t T,
                      uint16_t* x_out, float* out_last, void* ws, size_t ws_bytes, void* stream);

/* Expert-cache mode (first page, section "How a 125B model fits in 12 GB"; the
 * aireport.net page: an adaptive GPU cache of the most used experts, the others
 * computed elsewhere).  slot_of int32 [n_layers x E]: cache slot of expert e of
 * layer l, or -1; slot_pool: a bank whose expert s is the weights of slot s.
 * Routing uses L's router; gates are renormalised over all k selected experts.
 * out fp32 [T x H] = sum over selected experts WITH a slot of g * FFN + shared
 * expert; miss_rows int32 [T*k] receives the entries r = t*k + i whose expert has
 * no slot, ascending, and n_miss (device int32) their count. */
int moe_layer_forward_cached(const moe_layer_t* L, int32_t layer_idx, int32_t n_layers,
                             const int32_t* slot_of, const moe_bank_t* slot_pool,
                             const uint16_t* x, int32_t T, float* out,
                             int32_t* topk_ids, float* topk_gates,
                             int32_t* miss_rows, int32_t* n_miss,
                             void* ws, size_t ws_bytes, void* stream);

/* Host miss tier (first page, section "How a 125B model fits in 12 GB": every expert
 * is also held in system RAM, and the CPU computes a selected expert the GPU cache
 * lacks at the same time as the GPU computes the cached ones; the aireport.net page
 * names AVX-512 and AVX2 kernels for it).
 *
 * moe_cpu_expert_ffn takes HOST pointers only and makes no HIP call.  bank: a Q2 or
 * Q3 bank (layout as above) in host memory.  x bf16 [T x H]; ids int32 [T*k] and
 * gates fp32 [T*k] as the router writes them; rows int32 [n_rows]: entries
 * r = t*k + i, strictly ascending, each below T*k (a miss list).  y fp32 [T x H] is
 * overwritten: y[t] = sum over the listed entries r of token t, in ascending r, of
 * gates[r] * FFN_{ids[r]}(x[t]); tokens with no listed entry get zero rows.
 * n_threads: worker threads (0: three quarters of min(16, the host's hardware threads)).
 * Arithmetic: fp32 on AVX-512 where the CPU has AVX-512F/BW/VL/DQ, else AVX2 + FMA.
 * The result does not depend on n_threads.  Blocks until done; concurrent calls
 * are serialised.  MOE_EINVAL for bad arguments (unsorted rows, an id outside the
 * bank), MOE_EUNSUPPORTED for a bf16 bank or a CPU without AVX2. */
int moe_cpu_expert_ffn(const moe_bank_t* bank, const uint16_t* x, int32_t T, int32_t k,
                       const int32_t* ids, const float* gates, const int32_t* rows, int32_t n_rows,
                       float* y, int32_t n_threads);

/* Instruction set moe_cpu_expert_ffn uses on this CPU: 2 AVX-512, 1 AVX2, 0 none. */
int moe_cpu_isa(void);

/* Host bytes of the staging area moe_layer_forward_tiered needs for T tokens
 * (0 for invalid shapes). */
size_t moe_tiered_host_bytes(const moe_layer_t* L, int32_t T);

/* Tiered layer: the whole layer, with the cached experts on the GPU and the misses
 * on the host CPU, overlapped (same passage as moe_cpu_expert_ffn).  Arguments as
 * moe_layer_forward_cached, plus host_bank (all E routed experts of this layer in
 * host memory, the format of slot_pool), host_ws (at least moe_tiered_host_bytes
 * of pinned host memory, e.g. from hipHostMalloc) and n_threads (as above).
 * Order of work: routing and the miss list on the GPU; their copy to host_ws; the
 * cached experts, shared expert and combine on the GPU while the host computes the
 * misses with moe_cpu_expert_ffn; the misses' sum copied back and added.  On return
 * out (device, after the stream's work) = the full layer: every selected expert and
 * the shared expert; miss_rows / n_miss hold the miss list as in
 * moe_layer_forward_cached.  Blocks the calling thread until the miss sum has been
 * computed and its upload and add are enqueued; not capturable into a graph.  The
 * miss sum is staged in the workspace; host_ws must not be shared by overlapping
 * calls. */
int moe_layer_forward_tiered(const moe_layer_t* L, int32_t layer_idx, int32_t n_layers,
                             const int32_t* slot_of, const moe_bank_t* slot_pool,
                             const moe_bank_t* host_bank, const uint16_t* x, int32_t T, float* out,
                             int32_t* topk_ids, float* topk_gates,
                             int32_t* miss_rows, int32_t* n_miss,
                             void* ws, size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                             int32_t n_threads, void* stream);

/* Adaptive expert cache (first page, section "How a 125B model fits in 12 GB": the
 * cache of hot experts adapts to the conversation; the aireport.net page: the few
 * thousand most used experts, learned while chatting; every expert stays in pinned
 * system RAM).  The pages give no policy; the library's reading: decayed usage
 * counts per (layer, expert), each layer's cache periodically re-selected as its
 * most used experts, and slots refilled from host memory in the background.
 *
 * moe_expert_usage: counts uint32 [E] (device) = (counts >> decay_shift) + the number
 * of entries of topk_ids int32 [n_ids] (device) equal to e; ids outside [0, E) are
 * ignored.  E <= 1024, 0 <= decay_shift <= 31.  Exact (integer); one launch. */
int moe_expert_usage(const int32_t* topk_ids, int32_t n_ids, int32_t E, uint32_t* counts,
                     int32_t decay_shift, void* stream);

/* moe_cache_plan (HOST pointers, no HIP call): the moves that make one layer's cache
 * its n_slots most used experts.  counts uint32 [E]; slot_row int32 [E]: the layer's
 * current slot of each expert or -1; layer_slots int32 [n_slots]: the pool slots the
 * layer owns (distinct; every slot in slot_row must be one of them, one expert each).
 * Wanted = the n_slots largest counts (ties: lower id).  Incoming = wanted experts
 * without a slot, by count descending (ties: lower id); targets = the layer's free
 * slots ascending, then the slots of resident unwanted experts by count ascending
 * (ties: lower id).  Move i puts incoming[i] into targets[i], for
 * i < min(|incoming|, |targets|, max_moves): move_experts / move_slots int32
 * [max_moves], *n_moves the count.  MOE_EINVAL for an inconsistent slot_row. */
int moe_cache_plan(const uint32_t* counts, const int32_t* slot_row, int32_t E,
                   const int32_t* layer_slots, int32_t n_slots, int32_t max_moves,
                   int32_t* move_experts, int32_t* move_slots, int32_t* n_moves);

/* moe_cache_refill: starts the moves (at most 64; move lists in HOST memory) of layer
 * layer_idx.  host_bank: the layer's E routed experts in host memory (allocate it
 * pinned, e.g. hipHostMalloc, or the copies are not asynchronous); slot_pool: the
 * device pool (same format, Q2 or Q3); slot_of int32 [n_layers x E] (device).
 * On ``stream``: unmaps every expert that sits in a target slot and every incoming
 * expert (their entries become misses).  On ``copy_stream`` (NULL: ``stream``), after
 * that: copies each incoming expert's tensors into its slot, then records
 * done_event (a caller-created hipEvent_t).  Returns without waiting. */
int moe_cache_refill(const moe_bank_t* host_bank, const moe_bank_t* slot_pool, int32_t* slot_of,
                     int32_t layer_idx, int32_t n_layers, int32_t E,
                     const int32_t* move_experts, const int32_t* move_slots, int32_t n_moves,
                     void* done_event, void* stream, void* copy_stream);

/* moe_cache_commit: on ``stream``, waits for done_event (if not NULL) and maps each
 * incoming expert to its slot (the same move lists, n_slots = the pool's slot
 * count).  Calls on ``stream`` between refill and commit see the moved experts as
 * misses; calls after the commit see them as hits. */
int moe_cache_commit(int32_t* slot_of, int32_t layer_idx, int32_t n_layers, int32_t E, int32_t n_slots,
                     const int32_t* move_experts, const int32_t* move_slots, int32_t n_moves,
                     void* done_event, void* stream);

/* Measurement support.  Arms start_event / stop_event (hipEvent_t, created by
 * the caller) for the NEXT launch of the named kernel by any call above, then
 * forgets them (one-shot).  The events are attached to that kernel's dispatch
 * (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is the kernel's own
 * execution time on the stream it runs on, as a kernel trace reports it, without
 * the dispatch gap in front of it.  Where the named step is two launches (the
 * small-batch router front end), the interval runs from the first one's start to
 * the second one's end.  If the step launches nothing, both events are recorded
 * on the stream back to back.  Returns MOE_EINVAL for an unknown kernel or one
 * event NULL and the other not; both NULL disarms.  Process-global and not
 * thread-safe: meant for benchmarks only. */
enum {
  MOE_KERNEL_ROUTER = 0,       /* router logits (GEMV or MFMA GEMM) */
  MOE_KERNEL_GATEUP_GEMV = 1,  /* dequant-GEMV gate/up + SwiGLU */
  MOE_KERNEL_DOWN_GEMV = 2,    /* dequant-GEMV down projection */
  MOE_KERNEL_GATEUP_GEMM = 3,  /* MFMA grouped GEMM gate/up + SwiGLU */
  MOE_KERNEL_DOWN_GEMM = 4,    /* MFMA grouped GEMM down projection */
  MOE_KERNEL_COUNT = 5
};
int moe_time_next_launch(int32_t kernel, void* start_event, void* stop_event);

/* Static description of a status code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

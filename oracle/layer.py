"""Oracle of the MoE layer in float64: routing, permutation, expert FFN, combine,
stack and expert-cache mode.  Test infrastructure only.

Pages (cited by title and section):
  [A] "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU at Up to 94
      Tokens/s" (aibacon.net): section "What it is" (48 layers of 512 experts,
      10 routed and one shared expert per token); section "How a 125B model fits
      in 12 GB" (10 of 512 experts per layer are touched per token; an expert
      cache on the GPU, misses computed elsewhere).
  [E] "Strata: a 125B AI model on your gaming PC" (asadwebs.com): model spec
      table (rows "Layers", "Experts", "Hidden dimension").
  [C] "Strata Runs a 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU at
      up to 93 Tokens per Second" (aireport.net): the GPU keeps routers and
      shared experts, an adaptive cache of the most used experts, and the CPU
      computes the experts the GPU does not hold.

The pages state the structure (how many experts, which are always on) but not
the router function, the gate normalisation, the FFN type or the tie rule.  The
readings taken here: softmax router over all experts, top-k by logit with ties
to the lower expert index, gates = softmax probabilities renormalised over the
selected k, SwiGLU experts without biases (SiLU(gate) * up, then down), shared
expert added with weight 1.
"""
import numpy as np

from .formats import bf16_to_f64, f64_to_bf16_bits, expert_matrices


# ---------------------------------------------------------------- routing [A "What it is"]

def router_logits(x_bits, wr_bits, bias=None):
    """l[t, e] = sum_h x[t, h] * Wr[e, h] (+ b[e]); x bf16 [T, H], Wr bf16 [E, H] row-major."""
    x = bf16_to_f64(x_bits)
    wr = bf16_to_f64(wr_bits)
    logits = x @ wr.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return logits


def softmax(logits):
    """p[t, e] = exp(l - max) / sum exp(l - max) over all experts of token t."""
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def rank_experts(logits):
    """Per token, expert indices ordered by (logit descending, index ascending)."""
    T, E = logits.shape
    idx = np.arange(E)
    order = np.empty((T, E), dtype=np.int64)
    for t in range(T):
        order[t] = np.lexsort((idx, -logits[t]))
    return order


def select_topk(logits, k):
    """ids [T, k] int32: the k largest logits, ties broken toward the lower expert index.
    Selecting on the logits selects the same set as selecting on the softmax
    probabilities (exp is increasing) without ties created by rounding exp."""
    return rank_experts(logits)[:, :k].astype(np.int32)


def topk_margin(logits, k):
    """Gap between the k-th and (k+1)-th largest logit of each token (inf when k == E)."""
    T, E = logits.shape
    if k >= E:
        return np.full(T, np.inf)
    s = -np.sort(-logits, axis=1)
    return s[:, k - 1] - s[:, k]


def renormalised_gates(logits, ids):
    """g[t, i] = p[t, ids[t, i]] / sum_j p[t, ids[t, j]] with p the softmax over all experts."""
    p = softmax(logits)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x_bits, wr_bits, k, bias=None):
    """(ids [T, k] int32, gates [T, k] f64, margin [T] f64, logits [T, E] f64)."""
    logits = router_logits(x_bits, wr_bits, bias)
    ids = select_topk(logits, k)
    return ids, renormalised_gates(logits, ids), topk_margin(logits, k), logits


# ---------------------------------------------------------------- permutation

def permute(ids, E, with_shared):
    """Stable counting sort of the routed entries r = t * k + i by expert.

    Groups 0..E-1 are the routed experts; group E is the shared expert, which
    holds entries r = T * k + t for every token t when ``with_shared``.
    Returns offsets [E + 2] (exclusive scan of the group sizes, offsets[E + 1] =
    number of entries), sorted_rows [n] (entry at each sorted position, entries
    of one group in ascending r) and row_to_sorted [n] (its inverse)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    group = list(ids.reshape(-1).astype(np.int64))
    if with_shared:
        group += [E] * T
    n = len(group)
    counts = np.zeros(E + 1, dtype=np.int64)
    for g in group:
        counts[g] += 1
    offsets = np.zeros(E + 2, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    sorted_rows = np.empty(n, dtype=np.int64)
    row_to_sorted = np.empty(n, dtype=np.int64)
    for r, g in enumerate(group):
        sorted_rows[fill[g]] = r
        row_to_sorted[r] = fill[g]
        fill[g] += 1
    return offsets.astype(np.int32), sorted_rows.astype(np.int32), row_to_sorted.astype(np.int32)


# ---------------------------------------------------------------- expert FFN

def silu(a):
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)).

    For a below about -709, exp(-a) overflows to inf and the quotient is -0.0,
    the exact limit of SiLU; the overflow is expected there and not reported."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(x, w_gate, w_up, w_down):
    """SwiGLU FFN of one expert on rows x [M, H] (float64):
    a = x Wg^T, b = x Wu^T (each [M, I]), h = SiLU(a) * b, y = h Wd^T ([M, H])."""
    a = x @ w_gate.T
    b = x @ w_up.T
    h = silu(a) * b
    return h @ w_down.T


def bank_expert_fn(fmt, tensors, H, I, index_of=None):
    """Callable e -> (Wg, Wu, Wd) dequantising expert e of a bank on demand.
    ``index_of`` maps an expert id to its position in the bank (identity if None)."""
    cache = {}

    def fn(e):
        j = e if index_of is None else index_of(e)
        if j not in cache:
            cache[j] = expert_matrices(fmt, tensors, H, I, j)
        return cache[j]
    return fn


# ---------------------------------------------------------------- whole layer [A "What it is", E spec table]

def layer_forward(x_bits, wr_bits, k, expert_fn, shared_fn=None, bias=None, residual_bits=None):
    """out[t] = sum_{i<k} g[t,i] * FFN_{ids[t,i]}(x[t]) + FFN_shared(x[t]) (+ residual[t]),
    summed in the order i = 0..k-1, then the shared expert, then the residual.

    expert_fn(e) and shared_fn() return dense (Wg, Wu, Wd).  Returns
    (out [T, H] f64, ids, gates, margin)."""
    x = bf16_to_f64(x_bits)
    ids, gates, margin, _ = route(x_bits, wr_bits, k, bias)
    T, H = x.shape
    y = np.zeros((T, k, H))
    for e in np.unique(ids):
        rows = np.argwhere(ids == e)           # (t, i) pairs that chose e
        y[rows[:, 0], rows[:, 1]] = expert_ffn(x[rows[:, 0]], *expert_fn(int(e)))
    out = np.zeros((T, H))
    for i in range(k):
        out += gates[:, i:i + 1] * y[:, i]
    if shared_fn is not None:
        out += expert_ffn(x, *shared_fn())
    if residual_bits is not None:
        out += bf16_to_f64(residual_bits)
    return out, ids, gates, margin


def combine(y_sorted, row_to_sorted, gates, with_shared, residual_bits=None):
    """out[t] = sum_i g[t,i] * y_sorted[row_to_sorted[t*k+i]] (+ y_sorted[row_to_sorted[T*k+t]])
    (+ residual[t]), in that order."""
    T, k = gates.shape
    out = np.zeros((T, y_sorted.shape[1]))
    for i in range(k):
        out += gates[:, i:i + 1] * y_sorted[row_to_sorted[np.arange(T) * k + i]]
    if with_shared:
        out += y_sorted[row_to_sorted[T * k + np.arange(T)]]
    if residual_bits is not None:
        out += bf16_to_f64(residual_bits)
    return out


def residual_bf16(x_bits, out):
    """Next layer's input in a stack: bf16(x + out), rounded to nearest even once."""
    return f64_to_bf16_bits(bf16_to_f64(x_bits) + out)


RMS_EPS = 1e-6


def rms_norm_bf16(x_bits, eps=RMS_EPS):
    """Parameter-free RMSNorm of each token row, rounded to bf16:
    x / sqrt(mean(x^2) + eps).  The MoE input of every layer of a stack (the
    pages describe 48 layers but not the normalisation around the MoE block;
    without one the residual stream of random-weight SwiGLU experts diverges)."""
    x = bf16_to_f64(x_bits)
    r = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return f64_to_bf16_bits(x / r)


def stack_step(x_bits, layer_fn):
    """One layer of a stack: x_{l+1} = bf16(x_l + MoE_l(RMSNorm(x_l))).
    layer_fn(xn_bits) returns the layer's MoE output (float64 [T, H])."""
    xn = rms_norm_bf16(x_bits)
    return residual_bf16(x_bits, layer_fn(xn)), xn


# ---------------------------------------------------------------- expert cache [A "How a 125B model fits", C]

def cached_layer_forward(x_bits, wr_bits, k, slot_row, slot_fn, shared_fn=None, bias=None):
    """Cache-hit part of a layer.  slot_row[e] is the cache slot of expert e or -1.

    Routing and gates are those of the full layer (renormalised over all k
    selected experts).  out[t] = sum over hit i of g[t,i] * FFN_slot(x[t]) +
    FFN_shared(x[t]); misses = ascending entries r = t*k+i whose expert has no
    slot.  Returns (out, ids, gates, misses int32)."""
    x = bf16_to_f64(x_bits)
    ids, gates, margin, _ = route(x_bits, wr_bits, k, bias)
    T, H = x.shape
    slot_row = np.asarray(slot_row)
    out = np.zeros((T, H))
    y = np.zeros((T, k, H))
    hit = slot_row[ids] >= 0
    for e in np.unique(ids[hit]):
        rows = np.argwhere(ids == e)
        y[rows[:, 0], rows[:, 1]] = expert_ffn(x[rows[:, 0]], *slot_fn(int(slot_row[e])))
    for i in range(k):
        out += np.where(hit[:, i:i + 1], gates[:, i:i + 1] * y[:, i], 0.0)
    if shared_fn is not None:
        out += expert_ffn(x, *shared_fn())
    misses = np.array([t * k + i for t in range(T) for i in range(k) if not hit[t, i]], dtype=np.int32)
    return out, ids, gates, misses, margin


# ---------------------------------------------------------------- adaptive cache [A "How a 125B model fits", C]
# The pages say the cache of hot experts adapts to the conversation; they give no
# policy.  Reading: decayed integer usage counts, each layer's cache re-selected as
# its most used experts.

def usage_update(counts, ids, E, shift):
    """counts[e] // 2**shift + (number of ids equal to e), in uint32; ids outside [0, E) ignored."""
    out = [int(c) >> shift for c in counts]
    for e in np.asarray(ids).reshape(-1).tolist():
        if 0 <= e < E:
            out[e] += 1
    return np.array(out, dtype=np.uint64).astype(np.uint32)


def cache_plan(counts, slot_row, layer_slots, max_moves):
    """Moves (expert, slot) that turn a layer's cache into its len(layer_slots) most used experts.

    wanted: the most used experts (ties to the lower id); incoming: wanted ones
    without a slot, most used first; targets: free slots in ascending order, then
    the slots of unwanted residents, least used first (ties to the lower id).
    Returns lists (experts, slots) of length min(len(incoming), len(targets), max_moves)."""
    E = len(counts)
    n_slots = len(layer_slots)
    ranked = sorted(range(E), key=lambda e: (-int(counts[e]), e))
    wanted = set(ranked[:n_slots])
    incoming = [e for e in ranked[:n_slots] if slot_row[e] < 0]
    used = {int(slot_row[e]) for e in range(E) if slot_row[e] >= 0}
    free = sorted(int(s) for s in layer_slots if int(s) not in used)
    unwanted = sorted((e for e in range(E) if slot_row[e] >= 0 and e not in wanted),
                      key=lambda e: (int(counts[e]), e))
    targets = free + [int(slot_row[e]) for e in unwanted]
    n = min(len(incoming), len(targets), max_moves)
    return incoming[:n], targets[:n]


# ---------------------------------------------------------------- parity metric

def rel_max_err(got, ref):
    """max |got - ref| / sqrt(mean(ref^2)) over the whole output."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) / rms)

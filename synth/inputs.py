"""Seeded random draws for every tensor of the MoE layer.

Every tensor has its own Philox stream, keyed by (workload seed, tensor kind,
layer, index, attempt), so any single expert, token or layer can be regenerated
without materialising the rest (a 48-layer stack is 37.9 GB).

What is drawn (the recipe):
  * activations x: N(0, 1), rounded to bf16 (round-to-nearest-even from fp32);
    each token has its own stream, and ``attempt`` selects a fresh sub-stream for
    a token that has to be redrawn;
  * router weight: N(0, 0.02) -> bf16, [E, H] row-major;
  * router bias (skewed workloads): Zipf popularity p_e proportional to
    r_e^(-s) with r = 1 + pi(e) for a seeded permutation pi, bias = ln(p_e),
    stored as fp32;
  * 2-bit and 3-bit code planes: uniform random bytes (so every code is iid
    uniform over its range);
  * block scales: |N(0, 0.02)| -> fp16;
  * unquantised expert weights: N(0, 0.02) -> bf16.

Nothing here knows how the bytes are laid out or what they mean; the byte
counts per expert are the only shape facts used.
"""
import numpy as np

__all__ = [
    "stream", "f32_to_bf16_bits", "activation_row", "activations", "router_weight", "zipf_ranks",
    "zipf_bias", "expert_tensors", "bank", "hot_slot_table", "expert_nbytes", "budget_per_layer",
    "budget_slot_table",
]

_KIND = {
    "x": 1, "router": 2, "zipf": 3,
    "w13": 4, "w13_scale": 5, "w2": 6, "w2_scale": 7, "w13_hi": 8, "w2_hi": 9,
}


def stream(seed, kind, layer=0, index=0, attempt=0):
    """Independent Philox generator for one tensor (or one token / expert)."""
    tag = (_KIND[kind] << 56) | ((layer & 0xFFF) << 44) | ((attempt & 0xFFF) << 32) | (index & 0xFFFFFFFF)
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, tag], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activation_row(seed, layer, t, H, attempt=0):
    """bf16 bits [H] of token t, from its own stream (a later attempt is a fresh draw)."""
    g = stream(seed, "x", layer, t, attempt)
    return f32_to_bf16_bits(g.standard_normal(H, dtype=np.float32))


def activations(seed, layer, T, H, attempts=None):
    """bf16 bits [T, H]; token t is drawn from its own stream (attempt attempts[t])."""
    out = np.empty((T, H), dtype=np.uint16)
    for t in range(T):
        out[t] = activation_row(seed, layer, t, H, 0 if attempts is None else int(attempts[t]))
    return out


def router_weight(seed, layer, E, H, std=0.02):
    g = stream(seed, "router", layer)
    return f32_to_bf16_bits(g.standard_normal((E, H), dtype=np.float32) * np.float32(std))


def zipf_ranks(seed, layer, E):
    """pi(e): the popularity rank (0 = most popular) of every expert."""
    return stream(seed, "zipf", layer).permutation(E)


def zipf_bias(seed, layer, E, s):
    r = 1.0 + zipf_ranks(seed, layer, E).astype(np.float64)
    p = r ** (-float(s))
    p /= p.sum()
    return np.log(p).astype(np.float32)


def expert_nbytes(fmt, H, I):
    """Byte sizes of the per-expert arrays: {name: nbytes}."""
    n13, n2 = 2 * I * H, H * I
    if fmt == "bf16":
        return {"w13": 2 * n13, "w2": 2 * n2}
    d = {"w13": n13 // 4, "w13_scale": 2 * (n13 // 32), "w2": n2 // 4, "w2_scale": 2 * (n2 // 32)}
    if fmt == "q3":
        d["w13_hi"] = n13 // 8
        d["w2_hi"] = n2 // 8
    elif fmt != "q2":
        raise ValueError(fmt)
    return d


def _scales(g, n, std=0.02):
    return np.abs(g.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float16).view(np.uint16)


def expert_tensors(seed, layer, expert, fmt, H, I):
    """One expert's arrays as flat numpy buffers (uint8 code planes, uint16 fp16/bf16 bits)."""
    out = {}
    for name, nb in expert_nbytes(fmt, H, I).items():
        g = stream(seed, name, layer, expert)
        if fmt == "bf16":
            out[name] = f32_to_bf16_bits(g.standard_normal(nb // 2, dtype=np.float32) * np.float32(0.02))
        elif name.endswith("_scale"):
            out[name] = _scales(g, nb // 2)
        else:
            out[name] = np.frombuffer(g.bytes(nb), dtype=np.uint8).copy()
    return out


def bank(seed, layer, fmt, experts, H, I, workers=8):
    """Arrays of several experts, concatenated expert-major in the order of ``experts``.
    Experts are drawn on ``workers`` threads (each expert has its own streams, so
    the result does not depend on the thread count)."""
    sizes = expert_nbytes(fmt, H, I)
    experts = list(experts)
    out = {}
    for name, nb in sizes.items():
        dt = np.uint8 if (fmt != "bf16" and not name.endswith("_scale")) else np.uint16
        out[name] = np.empty(len(experts) * nb // np.dtype(dt).itemsize, dtype=dt)

    def fill(j):
        t = expert_tensors(seed, layer, experts[j], fmt, H, I)
        for name, arr in t.items():
            n = arr.size
            out[name][j * n:(j + 1) * n] = arr

    if workers <= 1 or len(experts) < 4:
        for j in range(len(experts)):
            fill(j)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(experts))))
    return out


def hot_slot_table(seed, n_layers, E, per_layer):
    """slot_of [n_layers, E] int32: the per_layer most popular experts of each layer get slots
    layer*per_layer + rank, every other (layer, expert) is -1 (not resident)."""
    slot_of = np.full((n_layers, E), -1, dtype=np.int32)
    for l in range(n_layers):
        r = zipf_ranks(seed, l, E)
        hot = r < per_layer
        slot_of[l, hot] = l * per_layer + r[hot]
    return slot_of


def budget_per_layer(n_layers, slots):
    """Slots of each layer when a budget of ``slots`` is shared out evenly: slots // n_layers each, one more
    for the first slots % n_layers layers."""
    q, r = divmod(int(slots), int(n_layers))
    return np.array([q + (1 if l < r else 0) for l in range(n_layers)], dtype=np.int64)


def budget_slot_table(seed, n_layers, E, per_layer, stride=None):
    """slot_of [n_layers, E] int32 for per-layer slot counts: the per_layer[l] most popular experts of layer l
    get slots base[l] + rank.  base[l] = l * stride (a pool laid out for ``stride`` slots a layer) or, if stride
    is None, the running sum of per_layer (a packed pool)."""
    per_layer = np.asarray(per_layer, dtype=np.int64)
    base = np.arange(n_layers, dtype=np.int64) * stride if stride is not None else \
        np.concatenate([[0], np.cumsum(per_layer)[:-1]])
    slot_of = np.full((n_layers, E), -1, dtype=np.int32)
    for l in range(n_layers):
        r = zipf_ranks(seed, l, E)
        hot = r < per_layer[l]
        slot_of[l, hot] = base[l] + r[hot]
    return slot_of

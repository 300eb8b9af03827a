"""GPU parity of the 3-bit path and of the expert-cache mode (slot table, hit
outputs, per-token miss list) against the fp64 oracle, through the C ABI.
Bars: top-k sets bit-exact, miss list and count bit-exact, outputs within 1e-2
of the oracle relative to its RMS."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as OF
from oracle import layer as OL
from quantized_expert_ffn_02_amd import binding as B
from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
from tests import workloads as W
from tests.test_gpu_parity import assert_route_matches, host, run_layer

pytestmark = pytest.mark.gpu
OUT_TOL = 1e-2


@pytest.fixture(scope="module")
def pool():
    assert torch.cuda.is_available()
    slot_of, pool = W.cache_pool("cache")
    s = synth.CONFIGS["cache"].shape
    dpool = DeviceBank(s.fmt, synth.CONFIGS["cache"].slots, s.hidden, s.inter, pool)
    return slot_of, pool, dpool


@pytest.mark.parametrize("T", [1, 4, 16, 17, 64, 1024])
def test_q3_layer_forward(T):
    # a plain (uncached) 3-bit layer: all 512 experts resident (T = 1: the decode
    # down projection's one-token launch shape; T = 16: the largest decode batch;
    # T = 17: the first batch past the decode path, on the 32-row grouped GEMM;
    # T = 1,024: a prompt-sized batch, which 3-bit weights also run on 32-row tiles)
    hl = W.host_layer("cache")
    x, _ = W.activations_with_margin(hl, T)
    d = W.upload(hl)
    out, out_bf, ids, gates, margin, _ = run_layer(d, x, T)
    ref, ids_r, gates_r, m_r = hl.oracle_forward(x)
    assert_route_matches(ids, gates, hl.logits(x), hl.shape.top_k, f"q3 T={T}")
    err = OL.rel_max_err(out, ref)
    print(f"q3 layer T={T}: max|err|/rms = {err:.3e}")
    assert err <= OUT_TOL


def test_q3_gemm_extreme_activations():
    # 3-bit weights on the 32-row grouped GEMM (T = 64) with rows rescaled over bf16's
    # range (x1e5, x1e12, x2^-20, x2^-40, tiny blocks, one large value among tiny ones):
    # each row enters the fp16 products scaled by a power of two, undone in fp32.
    from tests.test_gpu_parity import _extreme_rows
    hl = W.host_layer("cache")
    T = 64
    x0, _ = W.activations_with_margin(hl, T)
    rows = list(range(3, 10))
    x = x0.copy()
    x[rows] = _extreme_rows(x0[rows], rows=range(7), H=hl.H)
    assert (OL.topk_margin(hl.logits(x), hl.shape.top_k) >= 1e-4).all()
    d = W.upload(hl)
    out, out_bf, ids, gates, margin, _ = run_layer(d, x, T)
    assert np.isfinite(out).all()
    assert_route_matches(ids, gates, hl.logits(x), hl.shape.top_k, "q3 extreme")
    ref, *_ = hl.oracle_forward(x)
    for t in range(T):
        err = OL.rel_max_err(out[t], ref[t])
        if t in rows:
            print(f"q3 extreme row {t}: max|err|/rms = {err:.3e}")
        assert err <= OUT_TOL, f"row {t}"


@pytest.mark.parametrize("layer", [0, 17, 47])
def test_cached_layer(pool, layer):
    slot_of, hpool, dpool = pool
    w = synth.CONFIGS["cache"]
    s = w.shape
    T, k, E = w.tokens[0], s.top_k, s.n_experts
    hl = W.cache_layer("cache", layer, hpool)
    x, _ = W.activations_with_margin(hl, T)
    sb = DeviceBank(s.fmt, 1, s.hidden, s.inter, hl.shared)
    dl = DeviceLayer(s.hidden, E, k, s.inter, hl.wr, hl.bias, dpool, sb)
    ws = dl.workspace(T)
    out = torch.empty((T, s.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_slot = to_device(slot_of)
    B.layer_forward_cached(dl.struct, layer, w.layers, d_slot, dpool.struct, to_device(x), T, out, ids, gates,
                           miss, n_miss, ws)
    torch.cuda.synchronize()
    smat = OF.expert_matrices(s.fmt, hl.shared, s.hidden, s.inter)
    slot_fn = lambda sl: OF.expert_matrices(s.fmt, hpool, s.hidden, s.inter, sl)
    ref, ids_r, gates_r, misses_r, _ = OL.cached_layer_forward(x, hl.wr, k, slot_of[layer], slot_fn, lambda: smat,
                                                                bias=hl.bias)
    assert_route_matches(host(ids), host(gates), hl.logits(x), k, f"cache layer {layer}")
    nm = int(host(n_miss)[0])
    assert nm == len(misses_r)
    np.testing.assert_array_equal(host(miss)[:nm], misses_r)
    assert (host(miss)[nm:] == -7).all()                      # nothing written past the count
    err = OL.rel_max_err(host(out), ref)
    hits = T * k - nm
    print(f"cache layer {layer}: hits {hits}/{T * k}, max|err|/rms = {err:.3e}")
    assert err <= OUT_TOL


def _tiered(pool, layer, T, slot_of):
    """Tiered layer through the C ABI with the full host bank of the layer, and the oracle's full layer."""
    _, hpool, dpool = pool
    w = synth.CONFIGS["cache"]
    s = w.shape
    k, E, H, I = s.top_k, s.n_experts, s.hidden, s.inter
    hl = W.cache_layer("cache", layer, hpool)
    x, _ = W.activations_with_margin(hl, T)
    full = synth.bank(w.seed, layer, s.fmt, range(E), H, I)     # every routed expert of the layer, host memory
    hbank = B.make_host_bank(s.fmt, E, H, I, full)
    sb = DeviceBank(s.fmt, 1, H, I, hl.shared)
    dl = DeviceLayer(H, E, k, I, hl.wr, hl.bias, dpool, sb)
    ws = dl.workspace(T)
    host_ws = torch.empty(B.tiered_host_bytes(dl.struct, T), dtype=torch.uint8, pin_memory=True)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"tiered layer {layer} T={T}", flush=True)
    B.layer_forward_tiered(dl.struct, layer, w.layers, to_device(slot_of), dpool.struct, hbank, to_device(x), T, out,
                           ids, gates, miss, n_miss, ws, host_ws)
    torch.cuda.synchronize()
    smat = OF.expert_matrices(s.fmt, hl.shared, H, I)
    ref, ids_r, gates_r, _ = OL.layer_forward(x, hl.wr, k, OL.bank_expert_fn(s.fmt, full, H, I), lambda: smat,
                                              bias=hl.bias)
    assert_route_matches(host(ids), host(gates), hl.logits(x), k, f"tiered layer {layer}")
    nm = int(host(n_miss)[0])
    want = np.flatnonzero(slot_of[layer][ids_r.reshape(-1)] < 0).astype(np.int32)
    assert nm == len(want)
    np.testing.assert_array_equal(host(miss)[:nm], want)
    err = OL.rel_max_err(host(out), ref)
    print(f"tiered layer {layer} T={T}: misses {nm}/{T * k} on the host, max|err|/rms = {err:.3e}")
    assert err <= OUT_TOL
    return nm


@pytest.mark.parametrize("layer,T", [(0, 64), (17, 4), (47, 1)])
def test_tiered_layer(pool, layer, T):
    # hits on the GPU + misses on the host CPU = the oracle's full layer
    _tiered(pool, layer, T, pool[0])


def test_tiered_layer_mostly_misses(pool):
    # only the 8 most popular experts of the layer keep their slots: most entries go to the host
    slot_of = pool[0].copy()
    layer = 5
    row = slot_of[layer]
    cached = np.flatnonzero(row >= 0)
    keep = cached[np.argsort(row[cached])[:8]]                # slots are given in order of popularity
    cut = np.full_like(row, -1)
    cut[keep] = row[keep]
    slot_of[layer] = cut
    nm = _tiered(pool, layer, 8, slot_of)
    assert nm >= 8 * 10 // 4                                  # Zipf routing: the top 8 still take over half


@pytest.mark.parametrize("budget", [1589, 3872])
def test_slot_budget(budget):
    # The pages' other cache sizes, shared out over 48 layers (1,589: 34 or 33 slots
    # a layer; 3,872: 81 or 80).  One layer's pool is built from the budget's table;
    # hits, misses and the output must match the oracle as at 3,072 slots.
    w = synth.CONFIGS["cache"]
    s = w.shape
    k, E, H, I = s.top_k, s.n_experts, s.hidden, s.inter
    layer = 40
    per = synth.budget_per_layer(w.layers, budget)
    table = synth.budget_slot_table(w.seed, w.layers, E, per)
    row = table[layer]
    order = np.argsort(synth.zipf_ranks(w.seed, layer, E))[:per[layer]]
    lpool = synth.bank(w.seed, layer, s.fmt, order, H, I)          # this layer's slots, in slot order
    local = np.where(row >= 0, row - row[row >= 0].min(), -1).astype(np.int32)
    slot_of = np.full_like(table, -1)
    slot_of[layer] = local
    dpool = DeviceBank(s.fmt, int(per[layer]), H, I, lpool)
    hl = W.cache_layer("cache", layer, lpool)
    T = w.tokens[0]
    x, _ = W.activations_with_margin(hl, T)
    dl = DeviceLayer(H, E, k, I, hl.wr, hl.bias, dpool, DeviceBank(s.fmt, 1, H, I, hl.shared))
    ws = dl.workspace(T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.layer_forward_cached(dl.struct, layer, w.layers, to_device(slot_of), dpool.struct, to_device(x), T, out, ids,
                           gates, miss, n_miss, ws)
    torch.cuda.synchronize()
    smat = OF.expert_matrices(s.fmt, hl.shared, H, I)
    slot_fn = lambda sl: OF.expert_matrices(s.fmt, lpool, H, I, sl)
    ref, ids_r, gates_r, misses_r, _ = OL.cached_layer_forward(x, hl.wr, k, local, slot_fn, lambda: smat,
                                                                bias=hl.bias)
    assert_route_matches(host(ids), host(gates), hl.logits(x), k, f"budget {budget}")
    nm = int(host(n_miss)[0])
    assert nm == len(misses_r)
    np.testing.assert_array_equal(host(miss)[:nm], misses_r)
    err = OL.rel_max_err(host(out), ref)
    print(f"slot budget {budget} (layer {layer}: {per[layer]} slots): hits {T * k - nm}/{T * k}, "
          f"max|err|/rms = {err:.3e}")
    assert err <= OUT_TOL


# ------------------------------------------------------------------ adaptive cache

@pytest.mark.parametrize("n_ids,E,shift", [(40, 512, 1), (81920, 512, 2), (7, 1024, 0), (0, 16, 31), (640, 256, 5)])
def test_expert_usage_counts(n_ids, E, shift):
    # decayed usage counts: bit-exact against the oracle's integer definition
    rng = np.random.default_rng(n_ids + E)
    ids = rng.integers(-2, E + 2, size=n_ids).astype(np.int32)       # a few ids outside [0, E)
    counts0 = rng.integers(0, 2 ** 32, size=E, dtype=np.uint64).astype(np.uint32)
    d_counts = to_device(counts0)
    B.expert_usage(to_device(ids) if n_ids else None, n_ids, E, d_counts, shift)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(d_counts).view(np.uint32), OL.usage_update(counts0, ids, E, shift))


def _pinned(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).pin_memory()


@pytest.mark.parametrize("fmt", ["q2", "q3"])
def test_cache_adapts(fmt):
    # A small layer (H = 512, I = 256, 32 experts, top-4 + shared, Zipf routing) with an
    # 8-slot pool that starts empty.  Each round: a cached call, usage counts from its
    # ids, a plan, refill on a second stream, commit.  After every round the pool
    # holds each mapped expert's exact bytes, the slot table is the oracle's plan
    # applied, and the next cached call matches the oracle with that table.
    H, I, E, k, n_slots, T = 512, 256, 32, 4, 8, 16
    shape = synth.LayerShape(H, E, k, I, True, fmt, 1.1)
    hl = W.host_layer("cache", shape=shape)
    host_t = {n: _pinned(v) for n, v in hl.routed.items()}
    g = host_t.get
    hbank = B.make_bank(fmt, E, H, I, g("w13"), g("w13_hi"), g("w13_scale"), g("w2"), g("w2_hi"), g("w2_scale"))
    per_expert = {n: len(v) // E for n, v in hl.routed.items()}
    dpool = DeviceBank(fmt, n_slots, H, I, {n: np.zeros(per_expert[n] * n_slots, dtype=v.dtype)
                                            for n, v in hl.routed.items()})
    dl = DeviceLayer(H, E, k, I, hl.wr, hl.bias, dpool, DeviceBank(fmt, 1, H, I, hl.shared))
    ws = dl.workspace(T)
    slot_of = torch.full((1, E), -1, dtype=torch.int32, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    layer_slots = np.arange(n_slots, dtype=np.int32)
    copy_stream = torch.cuda.Stream()
    smat = OF.expert_matrices(fmt, hl.shared, H, I)
    row_ref = np.full(E, -1, dtype=np.int32)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    hits = []
    for rnd in range(3):
        x, _ = W.activations_with_margin(hl, T, x_seed=100 + rnd)
        B.layer_forward_cached(dl.struct, 0, 1, slot_of, dpool.struct, to_device(x), T, out, ids, gates, miss,
                               n_miss, ws)
        B.expert_usage(ids, T * k, E, counts, 1)
        torch.cuda.synchronize()
        # the cached call against the oracle with the table it saw (slot -> expert from the reference
        # table; weights from the host bank, never from the device pool)
        expert_of = {int(sl): int(e) for e, sl in enumerate(row_ref) if sl >= 0}
        slot_fn = lambda sl: OF.expert_matrices(fmt, hl.routed, H, I, expert_of[sl])
        ref, _, _, misses_r, _ = OL.cached_layer_forward(x, hl.wr, k, row_ref, slot_fn, lambda: smat, bias=hl.bias)
        nm = int(host(n_miss)[0])
        np.testing.assert_array_equal(host(miss)[:nm], misses_r)
        assert OL.rel_max_err(host(out), ref) <= OUT_TOL
        hits.append(T * k - nm)
        # plan, refill, commit
        c_h = host(counts).view(np.uint32)
        me, ms = B.cache_plan(c_h, row_ref, layer_slots, 64)
        want = OL.cache_plan(c_h, row_ref, layer_slots, 64)
        assert me.tolist() == want[0] and ms.tolist() == want[1]
        ev = torch.cuda.Event()
        ev.record()                                   # creates the underlying hipEvent
        B.cache_refill(hbank, dpool.struct, slot_of, 0, 1, E, me, ms, ev.cuda_event,
                       copy_stream=copy_stream.cuda_stream)
        B.cache_commit(slot_of, 0, 1, E, n_slots, me, ms, ev.cuda_event)
        torch.cuda.synchronize()
        for e, s in zip(me.tolist(), ms.tolist()):
            row_ref[row_ref == s] = -1
            row_ref[e] = s
        np.testing.assert_array_equal(host(slot_of)[0], row_ref)
        for e in np.flatnonzero(row_ref >= 0):
            s = int(row_ref[e])
            for n, t in dpool.tensors.items():
                b = per_expert[n] * hl.routed[n].itemsize
                got = t.view(torch.uint8)[s * b:(s + 1) * b].cpu().numpy()
                np.testing.assert_array_equal(got, hl.routed[n].view(np.uint8)[e * b:(e + 1) * b])
    print(f"{fmt}: hits per round {hits} of {T * k}")
    assert hits[0] == 0 and hits[-1] > hits[0]


def test_cached_q2_pool_fp8_tiles():
    # A real-shape 2-bit layer (uniform router) in expert-cache mode with a 48-slot pool
    # holding experts 0..47: at 64 tokens its hit groups have one to four entries, so they
    # run as fp8 x fp4 tiles under the slot map, and the missed groups' tiles write
    # nothing but zero rows.  Route, miss list and output against the oracle's cached layer.
    hl = W.host_layer("decode")
    s = hl.shape
    H, I, E, k, T, n_slots = s.hidden, s.inter, s.n_experts, s.top_k, 64, 48
    per = {n: len(v) // E for n, v in hl.routed.items()}
    dpool = DeviceBank(s.fmt, n_slots, H, I, {n: np.ascontiguousarray(v[:per[n] * n_slots]) for n, v in hl.routed.items()})
    dl = DeviceLayer(H, E, k, I, hl.wr, hl.bias, dpool, DeviceBank(s.fmt, 1, H, I, hl.shared))
    slot_row = np.full(E, -1, dtype=np.int32)
    slot_row[:n_slots] = np.arange(n_slots, dtype=np.int32)
    x, _ = W.activations_with_margin(hl, T)
    ws = dl.workspace(T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.layer_forward_cached(dl.struct, 0, 1, to_device(slot_row[None, :]), dpool.struct, to_device(x), T, out, ids,
                           gates, miss, n_miss, ws)
    torch.cuda.synchronize()
    smat = OF.expert_matrices(s.fmt, hl.shared, H, I)
    slot_fn = lambda sl: OF.expert_matrices(s.fmt, hl.routed, H, I, sl)   # slot sl holds expert sl
    ref, ids_r, gates_r, misses_r, _ = OL.cached_layer_forward(x, hl.wr, k, slot_row, slot_fn, lambda: smat,
                                                                bias=hl.bias)
    assert_route_matches(host(ids), host(gates), hl.logits(x), k, "cached q2 pool")
    counts = np.bincount(host(ids).reshape(-1), minlength=E)[:n_slots]
    assert ((counts >= 1) & (counts <= 4)).sum() >= 20, counts
    nm = int(host(n_miss)[0])
    assert nm == len(misses_r) and nm < T * k
    np.testing.assert_array_equal(host(miss)[:nm], misses_r)
    err = OL.rel_max_err(host(out), ref)
    print(f"cached q2 pool: hits {T * k - nm}/{T * k} in {(counts > 0).sum()} groups, max|err|/rms = {err:.3e}")
    assert err <= OUT_TOL


@pytest.mark.parametrize("T", [8, 32])
def test_tiered_layer_q2_small(T):
    # 2-bit weights end to end through the tiered layer: a small layer (H = 512, I = 256,
    # 32 experts, top-4 + shared, Zipf routing) whose experts of popularity rank 2..9 are
    # cached on the GPU; the host computes the rest, the two most popular among them (so
    # every batch has misses).  T = 8 routes as a decode batch, T = 32 takes the 32-row
    # GEMM path.
    shape = synth.LayerShape(512, 32, 4, 256, True, "q2", 1.1)
    H, I, E, k = shape.hidden, shape.inter, shape.n_experts, shape.top_k
    hl = W.host_layer("cache", shape=shape)
    w = synth.CONFIGS["cache"]
    order = np.argsort(synth.zipf_ranks(w.seed, 0, E))[2:10]
    pool = synth.bank(w.seed, 0, "q2", order, H, I)
    slot_of = np.full((1, E), -1, dtype=np.int32)
    slot_of[0, order] = np.arange(8, dtype=np.int32)
    dpool = DeviceBank("q2", 8, H, I, pool)
    hbank = B.make_host_bank("q2", E, H, I, hl.routed)
    dl = DeviceLayer(H, E, k, I, hl.wr, hl.bias, dpool, DeviceBank("q2", 1, H, I, hl.shared))
    x, _ = W.activations_with_margin(hl, T)
    ws = dl.workspace(T)
    host_ws = torch.empty(B.tiered_host_bytes(dl.struct, T), dtype=torch.uint8, pin_memory=True)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"tiered q2 T={T}", flush=True)
    B.layer_forward_tiered(dl.struct, 0, 1, to_device(slot_of), dpool.struct, hbank, to_device(x), T, out, ids, gates,
                           miss, n_miss, ws, host_ws)
    torch.cuda.synchronize()
    ref, ids_r, _, _ = hl.oracle_forward(x)
    assert_route_matches(host(ids), host(gates), hl.logits(x), k, f"tiered q2 T={T}")
    nm = int(host(n_miss)[0])
    want = np.flatnonzero(slot_of[0][ids_r.reshape(-1)] < 0).astype(np.int32)
    np.testing.assert_array_equal(host(miss)[:nm], want)
    err = OL.rel_max_err(host(out), ref)
    print(f"tiered q2 T={T}: misses {nm}/{T * k} on the host, max|err|/rms = {err:.3e}")
    assert nm > 0 and err <= OUT_TOL


def test_cache_refill_moves_a_resident_expert():
    # Moving an expert that already has a slot to another slot unmaps its old one (an
    # expert never maps to two slots); experts not named keep their slots; the new slot
    # holds the expert's exact bytes.
    H, I, E, n_slots = 512, 256, 16, 4
    fmt = "q2"
    routed = synth.bank(9, 0, fmt, range(E), H, I)
    host_t = {n: _pinned(v) for n, v in routed.items()}
    g = host_t.get
    hbank = B.make_bank(fmt, E, H, I, g("w13"), g("w13_hi"), g("w13_scale"), g("w2"), g("w2_hi"), g("w2_scale"))
    per_expert = {n: len(v) // E for n, v in routed.items()}
    dpool = DeviceBank(fmt, n_slots, H, I, {n: np.zeros(per_expert[n] * n_slots, dtype=v.dtype)
                                            for n, v in routed.items()})
    row = np.full(E, -1, dtype=np.int32)
    row[3], row[5] = 0, 1
    slot_of = to_device(row.reshape(1, E))
    me, ms = np.array([3, 7], dtype=np.int32), np.array([2, 0], dtype=np.int32)   # 3: slot 0 -> 2; 7 into slot 0
    ev = torch.cuda.Event()
    ev.record()
    B.cache_refill(hbank, dpool.struct, slot_of, 0, 1, E, me, ms, ev.cuda_event)
    B.cache_commit(slot_of, 0, 1, E, n_slots, me, ms, ev.cuda_event)
    torch.cuda.synchronize()
    want = np.full(E, -1, dtype=np.int32)
    want[3], want[5], want[7] = 2, 1, 0
    np.testing.assert_array_equal(host(slot_of)[0], want)
    for e, s in ((3, 2), (7, 0)):
        for n, t in dpool.tensors.items():
            b = per_expert[n] * routed[n].itemsize
            np.testing.assert_array_equal(t.view(torch.uint8)[s * b:(s + 1) * b].cpu().numpy(),
                                          routed[n].view(np.uint8)[e * b:(e + 1) * b])

"""Benchmark of the quantized MoE layer on one MI355X.

Workload (the decode configuration): one real-shape MoE layer -- hidden 2,560,
512 experts, top-10 routed + 1 shared, SwiGLU experts with intermediate 640 in
2-bit 32-weight blocks with fp16 scales -- run on a decode step of T tokens
(default 4 = 1 token + 3 MTP drafts verified in one pass; T = 1 is reported
alongside).  One step = one moe_layer_forward (route, permute, expert FFNs,
shared expert, combine) on device-resident inputs.  To keep the 256 MB Infinity
Cache from serving the weights, steps rotate over ``--rotate`` distinct layers
(each with its own weights) and a pool of distinct token batches.

Prints one JSON line with the throughput, the dominant kernel's roofline
(algorithmic bytes / its average duration, measured with HIP events that the
runtime stamps from that kernel's own dispatch on its stream), and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


# HBM traffic of the decode gate/up kernel (T = 4, 44 x 10 blocks) from two
# rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; command and figures in the
# profiles/ counter summary), each scaled by what the counter reads for a plain
# 256 MiB device copy: FETCH_SIZE reads 131,084.5 KiB for 262,144 KiB read
# (factor 2.0), WRITE_SIZE 262,144 KiB for 262,144 KiB written (factor 1.0).
# Reported only while the kernel's sources are the ones that were counted.
GATEUP_TRAFFIC = {
    "sources": ["decode_mx.hip", "mx.h", "mfma.h", "device.h", "topk.h"],
    "sha256": "f75e173595fc17fd1309b182d6a02a8034a9017e5376e798c45c18d5fa4a9aa8",
    "fetch_kib": 22235.7, "fetch_scale": 262144.0 / 131084.5,
    "write_kib": 118.8, "write_scale": 1.0,
    "tokens": 4,
}


def counted_traffic(entry, T):
    """Bytes per launch from the stored counter runs, or None if the kernel changed or T differs."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_expert_ffn_02_amd", "csrc")
    for f in entry["sources"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != entry["sha256"] or T != entry["tokens"]:
        return None
    return 1024.0 * (entry["fetch_kib"] * entry["fetch_scale"] + entry["write_kib"] * entry["write_scale"])


def q2_expert_bytes(H, I):
    """Bytes of one 2-bit expert: 3*H*I codes at 2 bits + one fp16 scale per 32 weights."""
    w = 3 * H * I
    return w // 4 + (w // 32) * 2


def gateup_bytes_per_expert(H, I):
    w = 2 * H * I
    return w // 4 + (w // 32) * 2


def cpu_baseline(hl_args, T, seconds):
    """The fp64 oracle (tests' reference implementation, untuned) on a bounded sample, single-threaded:
    BLAS limited to one thread and the process pinned to one core for the duration (restored after)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import formats as OF
    from oracle import layer as OL
    seed, shape, wr, routed, shared = hl_args
    H, I, k = shape.hidden, shape.inter, shape.top_k
    n_cpus = os.cpu_count() or 1
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        with threadpool_limits(limits=1):
            smat = OF.expert_matrices(shape.fmt, shared, H, I)
            threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
            t0 = time.perf_counter()
            tokens, batches = 0, 0
            while True:
                x = synth.activations(seed + 7000, batches, T, H)
                fn = OL.bank_expert_fn(shape.fmt, routed, H, I)   # fresh: every used expert is dequantised again
                OL.layer_forward(x, wr, k, fn, lambda: smat)
                tokens += T
                batches += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
    finally:
        os.sched_setaffinity(0, set(allowed))
    return {"value": tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cores_note": f"1 core of {n_cpus} (process pinned to core {core}, {len(allowed)} allowed; "
                          f"BLAS threads during the run: {threads})",
            "cpu_model": _cpu_model(),
            "sample": f"{batches} decode batches of T={T} tokens on layer 0 of the decode workload (fp64 numpy, "
                      f"experts dequantised on demand), {el:.1f} s"}


def bench_prefill(steps):
    """One 8,192-token prefill chunk of a real-shape 2-bit layer with Zipf(1.1)-skewed routing."""
    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
    wl = synth.CONFIGS["prefill"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    T = wl.tokens[0]
    wr = synth.router_weight(wl.seed, 0, E, H)
    bias = synth.zipf_bias(wl.seed, 0, E, s.zipf)
    rb = DeviceBank(s.fmt, E, H, I, synth.bank(wl.seed, 0, s.fmt, range(E), H, I, workers=16))
    sb = DeviceBank(s.fmt, 1, H, I, synth.bank(wl.seed, 0, s.fmt, [E], H, I))
    layer = DeviceLayer(H, E, k, I, wr, bias, rb, sb)
    xs = [to_device(synth.activations(wl.seed + 9000, j, T, H)) for j in range(2)]
    ws = layer.workspace(T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    for i in range(3):
        B.layer_forward(layer.struct, xs[i % 2], T, out, ws, topk_ids=ids)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        B.layer_forward(layer.struct, xs[i % 2], T, out, ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kev = {}
    # a prompt-sized chunk runs every group on the MFMA GEMM (no GEMV launches)
    for kern in (B.KERNEL_ROUTER, B.KERNEL_GATEUP_GEMM, B.KERNEL_DOWN_GEMM):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record()
            b.record()
        kev[kern] = evs
    torch.cuda.synchronize()
    for i in range(steps):
        for kern, evs in kev.items():
            B.time_next_launch(kern, evs[i][0].cuda_event, evs[i][1].cuda_event)
        B.layer_forward(layer.struct, xs[i % 2], T, out, ws, topk_ids=ids)
    torch.cuda.synchronize()
    kms = {kern: float(np.mean([a.elapsed_time(b) for a, b in evs])) for kern, evs in kev.items()}
    ids_h = ids.cpu().numpy()
    counts = np.bincount(ids_h.reshape(-1), minlength=E)
    # algorithmic FLOPs: router 2*T*H*E + every (token, expert) pair incl. the shared one: 6*H*I each
    flops = 2.0 * T * H * E + T * (k + 1) * 6.0 * H * I
    # a prompt-sized chunk (T >= 1024) sends every non-empty group to the GEMM,
    # smaller batches the groups of 32 or more entries
    big = counts >= (1 if T >= 1024 else 32)
    gemm_rows = int(counts[big].sum()) + T        # shared expert rows all go to the GEMM
    gemm_flops_gu = gemm_rows * 4.0 * H * I
    gemm_flops_dn = gemm_rows * 2.0 * H * I
    return {
        "workload": f"prefill: one 8,192-token chunk, real-shape 2-bit layer, Zipf(1.1) routing",
        "tokens": T, "layer_ms": ms, "tokens_per_s": T / (ms * 1e-3),
        "TFLOPs": flops / (ms * 1e-3) / 1e12,
        "mfma_frac_of_fp16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "algorithmic_GFLOP": flops / 1e9,
        "experts_on_gemm": int(big.sum()), "experts_empty": int((counts == 0).sum()),
        "kernel_us": {"router": kms[B.KERNEL_ROUTER] * 1e3, "gateup_gemm": kms[B.KERNEL_GATEUP_GEMM] * 1e3,
                      "down_gemm": kms[B.KERNEL_DOWN_GEMM] * 1e3},
        "gateup_gemm_TFLOPs": gemm_flops_gu / (kms[B.KERNEL_GATEUP_GEMM] * 1e-3) / 1e12,
        "down_gemm_TFLOPs": gemm_flops_dn / (kms[B.KERNEL_DOWN_GEMM] * 1e-3) / 1e12,
    }


def q3_expert_bytes(H, I):
    w = 3 * H * I
    return w // 4 + w // 8 + (w // 32) * 2


def bench_stack(steps):
    """48 independent real-shape 2-bit layers (37.9 GB resident), pre-norm residual chain,
    batch 1 and 32 x 4 = 128 verify tokens; eager calls and one HIP graph per step."""
    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
    wl = synth.CONFIGS["stack"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    layers = []
    for l in range(wl.layers):
        wr = synth.router_weight(wl.seed, l, E, H)
        bias = synth.zipf_bias(wl.seed, l, E, s.zipf)
        rb = DeviceBank(s.fmt, E, H, I, synth.bank(wl.seed, l, s.fmt, range(E), H, I, workers=16))
        sb = DeviceBank(s.fmt, 1, H, I, synth.bank(wl.seed, l, s.fmt, [E], H, I))
        layers.append(DeviceLayer(H, E, k, I, wr, bias, rb, sb))
    structs = [d.struct for d in layers]
    res = {"workload": "stack: 48 independent real-shape 2-bit layers, x_{l+1} = x_l + MoE_l(RMSNorm(x_l)), "
                       "Zipf(1.1) routing per layer", "resident_GB": sum(d.routed.nbytes() + d.shared.nbytes()
                                                                         for d in layers) / 1e9}
    for T in wl.tokens:
        x0 = to_device(synth.activations(wl.seed + 11000, 0, T, H))
        ws = layers[0].workspace(T)
        x_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        # bytes: per layer router + unique routed experts + shared, from one instrumented pass
        uniq = []
        cur = x0
        for d in layers:
            ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
            out = torch.empty((T, H), dtype=torch.float32, device="cuda")
            nxt = torch.empty((T, H), dtype=torch.int16, device="cuda")
            xn = torch.empty((T, H), dtype=torch.int16, device="cuda")
            B.rmsnorm_bf16(cur, T, H, xn)
            B.layer_forward(d.struct, xn, T, out, ws, residual=cur, out_bf16=nxt, topk_ids=ids)
            uniq.append(len(np.unique(ids.cpu().numpy())))
            cur = nxt
        step_bytes = sum(E * H * 2 + E * 4 + (u + 1) * q2_expert_bytes(H, I) for u in uniq) + 2 * T * H * 2
        for _ in range(3):
            B.stack_forward(structs, x0, T, x_out, ws)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            B.stack_forward(structs, x0, T, x_out, ws)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        # the same step captured once into a HIP graph and replayed
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            B.stack_forward(structs, x0, T, x_out, ws)
        g.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms_g = t0.elapsed_time(t1) / steps
        best = min(ms, ms_g)
        # algorithmic FLOPs per step: router 2*T*H*E and 6*H*I per (token, expert) incl. the shared one, per layer
        step_flops = wl.layers * (2.0 * T * H * E + T * (k + 1) * 6.0 * H * I)
        # the binding roofline: bytes at 8 TB/s against FLOPs at 2.5 PF (ridge about 315 flop/B)
        bound = "mfma" if step_flops / step_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
        tflops = step_flops / (best * 1e-3) / 1e12
        res[f"T{T}"] = {"step_ms_eager": ms, "step_ms_graph": ms_g, "tokens_per_s": T / (best * 1e-3),
                        "avg_unique_experts_per_layer": float(np.mean(uniq)), "algorithmic_GB_per_step":
                        step_bytes / 1e9, "sustained_GBps": step_bytes / (best * 1e-3) / 1e9,
                        "hbm_frac": step_bytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "algorithmic_GFLOP_per_step": step_flops / 1e9, "TFLOPs": tflops,
                        "mfma_frac_of_fp16_peak": tflops / MFMA_BF16_PEAK_TFLOPS, "bound": bound,
                        "roofline_frac": (tflops / MFMA_BF16_PEAK_TFLOPS) if bound == "mfma" else
                        step_bytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del g
    del layers
    torch.cuda.empty_cache()
    return res


def bench_cache(steps):
    """3-bit layer with a 3,072-slot expert cache (top 64 experts of each of 48 layers), 64 tokens,
    layer index swept over all 48 layers."""
    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
    wl = synth.CONFIGS["cache"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    T = wl.tokens[0]
    # One pool serves every slot budget: each layer's `stride` most popular experts, layer-major; a budget's
    # slot table maps a prefix of each layer's run (the pages' 1,589 and 3,872, and this workload's 3,072).
    budgets = {n: synth.budget_per_layer(wl.layers, n) for n in synth.CACHE_SLOT_BUDGETS}
    stride = int(max(int(p.max()) for p in budgets.values()))
    tables = {n: synth.budget_slot_table(wl.seed, wl.layers, E, p, stride=stride) for n, p in budgets.items()}
    slot_of = tables[wl.slots]
    parts = []
    for l in range(wl.layers):
        order = np.argsort(synth.zipf_ranks(wl.seed, l, E))[:stride]
        parts.append(synth.bank(wl.seed, l, s.fmt, order, H, I, workers=16))
    pool = DeviceBank(s.fmt, wl.layers * stride, H, I, {n: np.concatenate([p[n] for p in parts]) for n in parts[0]})
    del parts
    layers = []
    for l in range(wl.layers):
        wr = synth.router_weight(wl.seed, l, E, H)
        bias = synth.zipf_bias(wl.seed, l, E, s.zipf)
        sb = DeviceBank(s.fmt, 1, H, I, synth.bank(wl.seed, l, s.fmt, [E], H, I))
        layers.append(DeviceLayer(H, E, k, I, wr, bias, pool, sb))
    d_slot = to_device(slot_of)
    xs = [to_device(synth.activations(wl.seed + 12000, j, T, H)) for j in range(8)]
    ws = layers[0].workspace(T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((wl.layers, T, k), dtype=torch.int32, device="cuda")
    miss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nmiss = torch.empty(wl.layers, dtype=torch.int32, device="cuda")
    for l in range(wl.layers):
        B.layer_forward_cached(layers[l].struct, l, wl.layers, d_slot, pool.struct, xs[l % 8], T, out, ids[l], None,
                               miss, nmiss[l:l + 1], ws)
    torch.cuda.synchronize()
    ids_h, nm = ids.cpu().numpy(), nmiss.cpu().numpy()
    hit_bytes = []
    for l in range(wl.layers):
        u = np.unique(ids_h[l])
        hits = int((slot_of[l][u] >= 0).sum())
        hit_bytes.append(E * H * 2 + E * 4 + (hits + 1) * q3_expert_bytes(H, I))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    n = 0
    for _ in range(steps):
        for l in range(wl.layers):
            B.layer_forward_cached(layers[l].struct, l, wl.layers, d_slot, pool.struct, xs[l % 8], T, out, None,
                                   None, miss, nmiss[l:l + 1], ws)
            n += 1
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    gb = float(np.mean(hit_bytes))
    res = {"workload": "cache: real-shape 3-bit layer, 3,072-slot expert cache (top 64 of 512 per layer x 48 "
                       "layers, 6.6 GB), Zipf(1.1) routing, 64 tokens, layer index swept over 48 layers",
           "layer_us": ms * 1e3, "tokens_per_s": T / (ms * 1e-3), "hit_rate": 1 - float(nm.mean()) / (T * k),
           "algorithmic_MB_per_call": gb / 1e6, "GBps": gb / (ms * 1e-3) / 1e9,
           "hbm_frac": gb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    res["slot_budgets"] = {}
    for nb, table in tables.items():
        dt = to_device(table)
        for l in range(wl.layers):
            B.layer_forward_cached(layers[l].struct, l, wl.layers, dt, pool.struct, xs[l % 8], T, out, ids[l], None,
                                   miss, nmiss[l:l + 1], ws)
        torch.cuda.synchronize()
        ids_b, nm_b = ids.cpu().numpy(), nmiss.cpu().numpy()
        mb = float(np.mean([E * H * 2 + E * 4 + (int((table[l][np.unique(ids_b[l])] >= 0).sum()) + 1) *
                            q3_expert_bytes(H, I) for l in range(wl.layers)]))
        t0.record()
        n = 0
        for _ in range(steps):
            for l in range(wl.layers):
                B.layer_forward_cached(layers[l].struct, l, wl.layers, dt, pool.struct, xs[l % 8], T, out, None,
                                       None, miss, nmiss[l:l + 1], ws)
                n += 1
        t1.record()
        torch.cuda.synchronize()
        msb = t0.elapsed_time(t1) / n
        res["slot_budgets"][str(nb)] = {
            "slots": nb, "cache_GB": nb * q3_expert_bytes(H, I) / 1e9, "hit_rate": 1 - float(nm_b.mean()) / (T * k),
            "layer_us": msb * 1e3, "algorithmic_MB_per_call": mb / 1e6, "GBps": mb / (msb * 1e-3) / 1e9}
    res["tiered"] = bench_tiered(layers, pool, d_slot, xs, ws, wl)
    del layers, pool
    torch.cuda.empty_cache()
    return res


def bench_tiered(layers, pool, d_slot, xs, ws, wl, rounds=25, tier_layers=(0, 12, 24, 36)):
    """The cache workload's layers with the misses computed on the host (moe_layer_forward_tiered):
    every routed expert of 4 layers held in host memory; the host kernel also timed alone on the
    same miss lists.  Host wall-clock per call, each call ending in a stream synchronisation."""
    import time

    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    threads = max(1, min(16, os.cpu_count() or 1) * 3 // 4)   # the library's default
    banks = {l: synth.bank(wl.seed, l, s.fmt, range(E), H, I) for l in tier_layers}
    hb = {l: B.make_host_bank(s.fmt, E, H, I, banks[l]) for l in tier_layers}
    out = torch.empty((wl.tokens[0], H), dtype=torch.float32, device="cuda")
    res = {"host_layers": list(tier_layers), "host_bank_GB_per_layer": sum(v.nbytes for v in banks[0].values()) / 1e9,
           "isa": {2: "avx512", 1: "avx2"}.get(B.cpu_isa(), "none"), "threads": threads,
           "cpu": _cpu_model()}
    for T in (wl.tokens[0], 4):
        xt = [x[:T].contiguous() for x in xs]
        host_ws = torch.empty(B.tiered_host_bytes(layers[0].struct, T), dtype=torch.uint8, pin_memory=True)
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
        miss = torch.empty(T * k, dtype=torch.int32, device="cuda")
        nmiss = torch.empty(1, dtype=torch.int32, device="cuda")

        def tiered(l, j):
            B.layer_forward_tiered(layers[l].struct, l, wl.layers, d_slot, pool.struct, hb[l], xt[j % len(xt)], T,
                                   out, ids, gates, miss, nmiss, ws, host_ws, threads)

        def cached(l, j):
            B.layer_forward_cached(layers[l].struct, l, wl.layers, d_slot, pool.struct, xt[j % len(xt)], T, out,
                                   ids, gates, miss, nmiss, ws)

        # the miss lists of every (layer, batch) pair, for the host kernel alone
        lists = []
        for j, l in enumerate(tier_layers):
            cached(l, j)
            torch.cuda.synchronize()
            nm = int(nmiss.cpu()[0])
            lists.append((l, xt[j % len(xt)].cpu().numpy(), ids.cpu().numpy(), gates.cpu().numpy(),
                          miss.cpu().numpy()[:nm].copy()))
        timings = {}
        for name, fn in (("tiered", tiered), ("cached", cached)):
            for j, l in enumerate(tier_layers):
                fn(l, j)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = 0
            for _ in range(rounds):
                for j, l in enumerate(tier_layers):
                    fn(l, j)
                    torch.cuda.synchronize()
                    n += 1
            timings[name] = (time.perf_counter() - t0) / n
        y = np.empty((T, H), dtype=np.float32)
        t0 = time.perf_counter()
        for _ in range(rounds):
            for (l, x, i_, g_, rows) in lists:
                B.cpu_expert_ffn(hb[l], x, T, k, i_, g_, rows, len(rows), y, threads)
        cpu_s = (time.perf_counter() - t0) / (rounds * len(lists))
        misses = float(np.mean([len(t[4]) for t in lists]))
        res[f"T{T}"] = {"tiered_us": timings["tiered"] * 1e6, "cached_gpu_us": timings["cached"] * 1e6,
                        "host_kernel_us": cpu_s * 1e6, "misses_per_call": misses,
                        "host_Gweights_per_s": misses * 3 * H * I / cpu_s / 1e9 if misses else None}
    return res


def bench_adaptive(steps=320, period=8, shift_at=120, max_moves=16, slots=64, T=64):
    """Adaptive expert cache on one real-shape 3-bit layer (512 experts, 64 slots, 64-token batches, Zipf(1.1)
    routing): the cache starts as the first popularity order's top 64; at step ``shift_at`` the router's bias
    switches to another popularity order (a change of topic).  Every step adds its selections to decayed usage
    counts; every ``period`` steps the previous refill is committed and a new plan of at most ``max_moves`` moves
    is started on a copy stream from pinned host memory."""
    import time

    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
    wl = synth.CONFIGS["cache"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    layer = 0
    full = synth.bank(wl.seed, layer, s.fmt, range(E), H, I, workers=16)
    host_t = {n: torch.from_numpy(v.view(np.uint8)).pin_memory() for n, v in full.items()}
    g = host_t.get
    hbank = B.make_bank(s.fmt, E, H, I, g("w13"), g("w13_hi"), g("w13_scale"), g("w2"), g("w2_hi"), g("w2_scale"))
    order = np.argsort(synth.zipf_ranks(wl.seed, layer, E))[:slots]
    pool = DeviceBank(s.fmt, slots, H, I, synth.bank(wl.seed, layer, s.fmt, order, H, I))
    table0 = np.full((1, E), -1, dtype=np.int32)
    table0[0, order] = np.arange(slots, dtype=np.int32)
    wr = synth.router_weight(wl.seed, layer, E, H)
    sb = DeviceBank(s.fmt, 1, H, I, synth.bank(wl.seed, layer, s.fmt, [E], H, I))
    topics = [DeviceLayer(H, E, k, I, wr, synth.zipf_bias(wl.seed, lb, E, s.zipf), pool, sb) for lb in (layer, 100)]
    xs = [to_device(synth.activations(wl.seed + 13000, j, T, H)) for j in range(16)]
    ws = topics[0].workspace(T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    miss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nmiss = torch.zeros(steps, dtype=torch.int32, device="cuda")
    layer_slots = np.arange(slots, dtype=np.int32)
    copy_stream = torch.cuda.Stream()

    def run(adapt):
        slot_of = to_device(table0)
        counts = torch.zeros(E, dtype=torch.int32, device="cuda")
        pending, moved = None, 0
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for step in range(steps):
            L = topics[0 if step < shift_at else 1]
            B.layer_forward_cached(L.struct, 0, 1, slot_of, pool.struct, xs[step % 16], T, out, ids, gates, miss,
                                   nmiss[step:step + 1], ws)
            evs[step + 1].record()
            if adapt:
                B.expert_usage(ids, T * k, E, counts, 1 if step % period == 0 else 0)
            torch.cuda.current_stream().synchronize()        # a decode loop waits for each step's output
            if not adapt or step % period != period - 1:
                continue
            # one refill in flight, committed once its copies are done (the compute stream never waits
            # for them); the next plan is made after the commit
            if pending is not None:
                if not pending[2].query():
                    continue
                B.cache_commit(slot_of, 0, 1, E, slots, pending[0], pending[1], pending[2].cuda_event)
                pending = None
            me, ms = B.cache_plan(counts.cpu().numpy().view(np.uint32), slot_of.cpu().numpy()[0], layer_slots,
                                  max_moves)
            if len(me):
                ev = torch.cuda.Event()
                ev.record()
                B.cache_refill(hbank, pool.struct, slot_of, 0, 1, E, me, ms, ev.cuda_event,
                               copy_stream=copy_stream.cuda_stream)
                pending = (me, ms, ev)
                moved += len(me)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        hit = 1.0 - nmiss.cpu().numpy().astype(np.float64) / (T * k)
        # stream time per step (event to event) over the 40 steps before the shift and the last 40
        win = {"before_shift": evs[shift_at - 40].elapsed_time(evs[shift_at]) / 40 * 1e3,
               "last_40": evs[steps - 40].elapsed_time(evs[steps]) / 40 * 1e3}
        return dt, hit, moved, win

    run(False)                                            # warm-up
    static_s, static_hit, _, static_win = run(False)
    adapt_s, hit, moved, adapt_win = run(True)
    before = float(hit[shift_at - 40:shift_at].mean())
    target = 0.95 * before
    after = hit[shift_at:]
    rec = next((i for i in range(len(after) - 7) if after[i:i + 8].mean() >= target), None)
    # refill bandwidth on an idle GPU: 16 experts from pinned memory into their slots (the second of two
    # refills of the same experts: the first DMA from a pinned page costs extra)
    me = np.arange(16, dtype=np.int32) + 200
    ms = np.arange(16, dtype=np.int32)
    slot_of = to_device(table0)
    e0, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done.record(copy_stream)                              # creates the underlying hipEvent
    B.cache_refill(hbank, pool.struct, slot_of, 0, 1, E, me, ms, done.cuda_event, copy_stream=copy_stream.cuda_stream)
    torch.cuda.synchronize()
    e0.record(copy_stream)
    B.cache_refill(hbank, pool.struct, slot_of, 0, 1, E, me, ms, done.cuda_event, copy_stream=copy_stream.cuda_stream)
    torch.cuda.synchronize()
    refill_ms = e0.elapsed_time(done)
    refill_bytes = 16 * q3_expert_bytes(H, I)
    return {"workload": "adaptive cache: one real-shape 3-bit layer, 64 slots of 512 experts, 64-token batches, "
                        f"Zipf(1.1) routing whose popularity order changes at step {shift_at} of {steps}; each step waits for "
                        f"its output (as a decode loop does); re-plan every {period} steps (at most {max_moves} moves, "
                        "one refill in flight, committed once its copies are done), "
                        "refills from pinned host memory",
            "hit_rate_before_shift": before, "hit_rate_first_period_after": float(after[:period].mean()),
            "hit_rate_last_40_steps": float(hit[-40:].mean()),
            "hit_rate_last_40_steps_static": float(static_hit[-40:].mean()),
            "steps_to_recover_95pct": rec, "experts_moved": moved,
            "step_us_adaptive": adapt_s * 1e6, "step_us_static": static_s * 1e6,
            "stream_us_per_step_before_shift": {"adaptive": adapt_win["before_shift"],
                                                "static": static_win["before_shift"]},
            "stream_us_per_step_last_40": {"adaptive": adapt_win["last_40"], "static": static_win["last_40"]},
            "refill_16_experts_ms": refill_ms, "refill_GBps": refill_bytes / (refill_ms * 1e-3) / 1e9}


def bench_coder(steps, rotate=16):
    """The pruned "Coder" layer shape: 256 experts, top-10 + shared, 2-bit, same kernels; T = 1, 4 (decode)
    and 64 (the 32-row GEMM path), 16 distinct layers rotated."""
    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device
    wl = synth.CONFIGS["coder"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    layers = []
    for l in range(rotate):
        wr = synth.router_weight(wl.seed, l, E, H)
        rb = DeviceBank(s.fmt, E, H, I, synth.bank(wl.seed, l, s.fmt, range(E), H, I, workers=16))
        sb = DeviceBank(s.fmt, 1, H, I, synth.bank(wl.seed, l, s.fmt, [E], H, I))
        layers.append(DeviceLayer(H, E, k, I, wr, None, rb, sb))
    res = {"workload": "coder: real-shape 2-bit layer with 256 experts (the pruned build), top-10 + shared, "
                       f"{rotate} distinct layers rotated"}
    for T in wl.tokens:
        xs = [to_device(synth.activations(wl.seed + 7000, j, T, H)) for j in range(16)]
        ws = layers[0].workspace(T)
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        n_steps = steps if T <= 16 else max(steps // 10, 1)
        ids = torch.empty((n_steps, T, k), dtype=torch.int32, device="cuda")
        for i in range(50):
            B.layer_forward(layers[i % rotate].struct, xs[i % 16], T, out, ws)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(n_steps):
            B.layer_forward(layers[i % rotate].struct, xs[i % 16], T, out, ws, topk_ids=ids[i])
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / n_steps
        ids_h = ids.cpu().numpy()
        d = float(np.mean([len(np.unique(ids_h[i])) for i in range(n_steps)]))
        step_bytes = E * H * 2 + (d + 1) * q2_expert_bytes(H, I) + T * H * 2 + T * H * 4
        res[f"T{T}"] = {"layer_us": ms * 1e3, "tokens_per_s": T / (ms * 1e-3), "unique_experts_per_step": d,
                        "layer_GBps": step_bytes / (ms * 1e-3) / 1e9,
                        "layer_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del layers
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def progress(section):
    """One line on stderr per finished section (stdout carries only the JSON line)."""
    print(f"bench: {section} done", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--tokens", type=int, default=4)
    ap.add_argument("--rotate", type=int, default=16, help="distinct layers cycled through")
    ap.add_argument("--pool", type=int, default=64, help="distinct token batches cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--cache-steps", type=int, default=5)
    ap.add_argument("--no-cache", action="store_true")
    ap.add_argument("--coder-steps", type=int, default=2000)
    ap.add_argument("--no-coder", action="store_true")
    ap.add_argument("--no-adaptive", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run 10 plain device copies of BYTES bytes (a known-size reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from quantized_expert_ffn_02_amd import binding as B
    from quantized_expert_ffn_02_amd.device_layer import DeviceBank, DeviceLayer, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch scale the
        # counters of the kernels above to bytes
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = synth.CONFIGS["decode"]
    s = wl.shape
    H, I, E, k = s.hidden, s.inter, s.n_experts, s.top_k
    R, T = args.rotate, args.tokens

    layers, host0 = [], None
    for l in range(R):
        wr = synth.router_weight(wl.seed, l, E, H)
        routed = synth.bank(wl.seed, l, s.fmt, range(E), H, I, workers=16)
        shared = synth.bank(wl.seed, l, s.fmt, [E], H, I)
        rb = DeviceBank(s.fmt, E, H, I, routed)
        sb = DeviceBank(s.fmt, 1, H, I, shared)
        layers.append(DeviceLayer(H, E, k, I, wr, None, rb, sb))
        if l == 0:
            host0 = (wl.seed, s, wr, routed, shared)
        del routed
    pool = [to_device(synth.activations(wl.seed + 5000, j, T, H)) for j in range(args.pool)]
    progress("decode layer setup")

    def run(T_, steps, warm, time_kernels):
        """Headline loop (no events inside), then, if asked, a second loop with one-shot
        HIP events around the router, gate/up and down kernels of every step."""
        ws = layers[0].workspace(T_)
        out = torch.empty((T_, H), dtype=torch.float32, device="cuda")
        ids = torch.empty((max(steps, 1), T_, k), dtype=torch.int32, device="cuda")
        xs = pool if T_ == T else [to_device(synth.activations(wl.seed + 6000, j, T_, H)) for j in range(args.pool)]
        for i in range(warm):
            B.layer_forward(layers[i % R].struct, xs[i % len(xs)], T_, out, ws, topk_ids=ids[0])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            B.layer_forward(layers[i % R].struct, xs[i % len(xs)], T_, out, ws, topk_ids=ids[i])
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        ids_h = ids.cpu().numpy()
        uniq = np.array([len(np.unique(ids_h[i])) for i in range(steps)])
        kms = {}
        if time_kernels:
            kev = {}
            for kern in (B.KERNEL_ROUTER, B.KERNEL_GATEUP_GEMV, B.KERNEL_DOWN_GEMV):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(steps)]
                for a, b in evs:      # create the underlying hipEvents
                    a.record()
                    b.record()
                kev[kern] = evs
            torch.cuda.synchronize()
            for i in range(steps):
                for kern, evs in kev.items():
                    B.time_next_launch(kern, evs[i][0].cuda_event, evs[i][1].cuda_event)
                B.layer_forward(layers[i % R].struct, xs[i % len(xs)], T_, out, ws)
            torch.cuda.synchronize()
            kms = {kern: float(np.mean([a.elapsed_time(b) for a, b in evs])) for kern, evs in kev.items()}
        return ms, kms, uniq

    ms, kms, uniq = run(T, args.steps, args.warmup, True)
    ms_step = ms / args.steps
    d_avg = float(uniq.mean())
    eb = q2_expert_bytes(H, I)
    step_bytes = E * H * 2 + (d_avg + 1) * eb + T * H * 2 + T * H * 4
    gu_bytes = (d_avg + 1) * gateup_bytes_per_expert(H, I) + T * H * 2 + (T * k + T) * I * 4
    gu_ms = kms[B.KERNEL_GATEUP_GEMV]
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    # T = 1 alongside (same layers, no kernel events)
    ms1, _, uniq1 = run(1, max(args.steps // 2, 1), args.warmup, False)
    ms1_step = ms1 / max(args.steps // 2, 1)
    step_bytes1 = E * H * 2 + (float(uniq1.mean()) + 1) * eb + H * 2 + H * 4
    # an MTP verify batch of 32 sequences x (1 + 3 drafts): 128 independent tokens on the
    # same layers (the 32-row grouped GEMM path)
    verify = None
    if not args.no_verify:
        TV, sv = 128, max(args.steps // 10, 1)
        msv, _, uniqv = run(TV, sv, max(args.warmup // 10, 5), False)
        msv_step = msv / sv
        dv = float(uniqv.mean())
        bytes_v = E * H * 2 + (dv + 1) * eb + TV * H * 2 + TV * H * 4
        flops_v = 2.0 * TV * H * E + TV * (k + 1) * 6.0 * H * I
        gbps_v = bytes_v / (msv_step * 1e-3) / 1e9
        tflops_v = flops_v / (msv_step * 1e-3) / 1e12
        hbm_bound_v = flops_v / bytes_v < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        verify = {
            "workload": f"verify: one real-shape 2-bit layer, T={TV} independent tokens (32 sequences x (1 + 3 MTP "
                        f"drafts)), the decode layers and router, {R} distinct layers rotated",
            "layer_us": msv_step * 1e3,
            "tokens_per_s": TV / (msv_step * 1e-3),
            "unique_experts_per_step": dv,
            "algorithmic_MB_per_step": bytes_v / 1e6,
            "GBps": gbps_v,
            "hbm_frac": gbps_v / HBM_PEAK_GBS,
            "algorithmic_GFLOP_per_step": flops_v / 1e9,
            "TFLOPs": tflops_v,
            "mfma_frac_of_fp16_peak": tflops_v / MFMA_BF16_PEAK_TFLOPS,
            "bound": "hbm" if hbm_bound_v else "mfma",
            "roofline_frac": gbps_v / HBM_PEAK_GBS if hbm_bound_v else tflops_v / MFMA_BF16_PEAK_TFLOPS,
        }

    result = {
        "metric": "MoE-layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"decode: one real-shape 2-bit MoE layer, T={T} tokens (1 + 3 MTP drafts), "
                        f"{R} distinct layers rotated",
            "hidden": H, "experts": E, "top_k": k, "shared_experts": 1, "inter": I,
            "weights": "2-bit codes, 32-weight blocks, fp16 scales (1,536,000 B per expert)",
            "arithmetic": "2-bit codes enter the fp8 x fp4 block-scaled matrix cores exactly (fp4 c/2); bf16 x "
                          "and fp32 h enter as four fixed-point e4m3 pieces per 32-column block (within 2^-19 of "
                          "the block's largest magnitude); fp16 block scales applied in fp32; fp32 accumulation "
                          "and output",
            "tokens": T, "layers_rotated": R,
        },
        "decode": {
            "layer_us": ms_step * 1e3,
            "unique_experts_per_step": d_avg,
            "algorithmic_bytes_per_step": step_bytes,
            "layer_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
            "layer_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_us": {"router": kms[B.KERNEL_ROUTER] * 1e3, "gateup_gemv": gu_ms * 1e3,
                          "down_gemv": kms[B.KERNEL_DOWN_GEMV] * 1e3},
            "T1": {"tokens_per_s": 1 / (ms1_step * 1e-3), "layer_us": ms1_step * 1e3,
                   "layer_GBps": step_bytes1 / (ms1_step * 1e-3) / 1e9},
        },
        "roofline": {
            "kernel": "k_decode_gateup_mx (top-k, gate/up + SwiGLU on the fp8 x fp4 matrix cores, down-table epilogue)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counted_traffic(GATEUP_TRAFFIC, T),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_us": gu_ms * 1e3,
        },
    }
    if verify is not None:
        result["verify"] = verify
    del layers, pool
    torch.cuda.empty_cache()
    progress("decode and verify")
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args.prefill_steps)
        progress("prefill")
    if not args.no_stack:
        result["stack"] = bench_stack(args.stack_steps)
        progress("stack")
    if not args.no_cache:
        result["cache"] = bench_cache(args.cache_steps)
        progress("cache")
    if not args.no_coder:
        result["coder"] = bench_coder(args.coder_steps)
        progress("coder")
    if not args.no_adaptive:
        result["adaptive"] = bench_adaptive()
        progress("adaptive")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host0, T, args.cpu_seconds)
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
        progress("cpu baseline")
    print(json.dumps(result))


if __name__ == "__main__":
    main()

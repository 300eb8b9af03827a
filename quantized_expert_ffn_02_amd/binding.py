"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function here forwards to the C ABI with device pointers taken from torch
tensors and the current HIP stream; all computation happens in the library's
kernels.  There is no fallback: if libmoe.so is missing, ``lib()`` raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 40 << 20
FMT_NONE, FMT_BF16, FMT_Q2, FMT_Q3 = -1, 0, 1, 2
FMT_BY_NAME = {"bf16": FMT_BF16, "q2": FMT_Q2, "q3": FMT_Q3}
WS_CONTROL_BYTES = 65536
MAX_TOKENS = 8192
KERNEL_ROUTER, KERNEL_GATEUP_GEMV, KERNEL_DOWN_GEMV, KERNEL_GATEUP_GEMM, KERNEL_DOWN_GEMM = 0, 1, 2, 3, 4

# Every function the header declares, with (restype, argtypes).
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class Bank(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("w13", _vp), ("w13_hi", _vp), ("w13_scale", _vp),
        ("w2", _vp), ("w2_hi", _vp), ("w2_scale", _vp),
    ]


class Layer(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("w_router", _vp), ("router_bias", _vp),
        ("routed", Bank), ("shared", Bank),
    ]


_SIGS = {
    "moe_workspace_bytes": (_sz, [ctypes.POINTER(Layer), _i32]),
    "moe_workspace_clear": (ctypes.c_int, [_vp, _sz, _vp]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(Layer), _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_q2": (ctypes.c_int, [ctypes.POINTER(Layer), _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(Layer), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _sz, _vp]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Layer), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp]),
    "moe_stack_forward": (ctypes.c_int, [ctypes.POINTER(Layer), _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_layer_forward_cached": (ctypes.c_int, [ctypes.POINTER(Layer), _i32, _i32, _vp, ctypes.POINTER(Bank), _vp,
                                                _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_cpu_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Bank), _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _i32]),
    "moe_cpu_isa": (ctypes.c_int, []),
    "moe_tiered_host_bytes": (_sz, [ctypes.POINTER(Layer), _i32]),
    "moe_layer_forward_tiered": (ctypes.c_int, [ctypes.POINTER(Layer), _i32, _i32, _vp, ctypes.POINTER(Bank),
                                                ctypes.POINTER(Bank), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                _vp, _sz, _i32, _vp]),
    "moe_expert_usage": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp]),
    "moe_cache_plan": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp]),
    "moe_cache_refill": (ctypes.c_int, [ctypes.POINTER(Bank), ctypes.POINTER(Bank), _vp, _i32, _i32, _i32, _vp, _vp,
                                        _i32, _vp, _vp, _vp]),
    "moe_cache_commit": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp]),
    "moe_time_next_launch": (ctypes.c_int, [_i32, _vp, _vp]),
    "moe_rmsnorm_bf16": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}

_LIB = None


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_expert_ffn_02_amd.build`")
        # torch ships its own HIP runtime with the same soname; importing torch first
        # makes libmoe bind to that one instance, so torch streams are valid here
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def declared_functions():
    return sorted(_SIGS)


def strerror(code):
    return lib().moe_strerror(int(code)).decode()


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def ptr(t):
    """Device address of a tensor, or None for None."""
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------- structs

def make_bank(fmt, n_experts, hidden, inter, w13=None, w13_hi=None, w13_scale=None, w2=None, w2_hi=None,
              w2_scale=None):
    f = FMT_BY_NAME[fmt] if isinstance(fmt, str) else fmt
    return Bank(f, n_experts, hidden, inter, ptr(w13), ptr(w13_hi), ptr(w13_scale), ptr(w2), ptr(w2_hi),
                ptr(w2_scale))


def no_bank():
    return Bank(FMT_NONE, 0, 0, 0, None, None, None, None, None, None)


def make_layer(hidden, n_experts, top_k, inter, w_router, router_bias, routed, shared=None):
    return Layer(hidden, n_experts, top_k, inter, ptr(w_router), ptr(router_bias), routed,
                 shared if shared is not None else no_bank())


# ---------------------------------------------------------------- calls

def workspace_bytes(layer, T):
    return int(lib().moe_workspace_bytes(ctypes.byref(layer), int(T)))


def workspace_clear(ws, stream=None):
    _check("moe_workspace_clear", lib().moe_workspace_clear(ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def route(layer, x, T, topk_ids, topk_gates, margin, ws, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(layer), ptr(x), int(T), ptr(topk_ids), ptr(topk_gates),
                                        ptr(margin), ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def permute(topk_ids, T, k, E, with_shared, offsets, sorted_rows, row_to_sorted, ws, stream=None):
    _check("moe_permute", lib().moe_permute(ptr(topk_ids), int(T), int(k), int(E), int(bool(with_shared)),
                                            ptr(offsets), ptr(sorted_rows), ptr(row_to_sorted), ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)))


def expert_ffn_q2(layer, x, T, offsets, sorted_rows, y_sorted, ws, stream=None):
    _check("moe_expert_ffn_q2", lib().moe_expert_ffn_q2(ctypes.byref(layer), ptr(x), int(T), ptr(offsets),
                                                        ptr(sorted_rows), ptr(y_sorted), ptr(ws),
                                                        ws.numel() * ws.element_size(), _stream(stream)))


def combine(y_sorted, row_to_sorted, topk_gates, T, k, H, with_shared, residual, out, out_bf16=None, stream=None):
    _check("moe_combine", lib().moe_combine(ptr(y_sorted), ptr(row_to_sorted), ptr(topk_gates), int(T), int(k),
                                            int(H), int(bool(with_shared)), ptr(residual), ptr(out), ptr(out_bf16),
                                            _stream(stream)))


def layer_forward(layer, x, T, out, ws, residual=None, out_bf16=None, topk_ids=None, topk_gates=None, margin=None,
                  stream=None):
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(layer), ptr(x), int(T), ptr(residual), ptr(out), ptr(out_bf16), ptr(topk_ids),
        ptr(topk_gates), ptr(margin), ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def layer_forward_noalloc(layer, x, T, out, residual=None, out_bf16=None, topk_ids=None, topk_gates=None,
                          margin=None, stream=None):
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(layer), ptr(x), int(T), ptr(residual), ptr(out), ptr(out_bf16), ptr(topk_ids),
        ptr(topk_gates), ptr(margin), _stream(stream)))


def stack_forward(layers, x0, T, x_out, ws, out_last=None, stream=None):
    arr = (Layer * len(layers))(*layers)
    _check("moe_stack_forward", lib().moe_stack_forward(arr, len(layers), ptr(x0), int(T), ptr(x_out),
                                                        ptr(out_last), ptr(ws), ws.numel() * ws.element_size(),
                                                        _stream(stream)))


def layer_forward_cached(layer, layer_idx, n_layers, slot_of, slot_pool, x, T, out, topk_ids, topk_gates,
                         miss_rows, n_miss, ws, stream=None):
    _check("moe_layer_forward_cached", lib().moe_layer_forward_cached(
        ctypes.byref(layer), int(layer_idx), int(n_layers), ptr(slot_of), ctypes.byref(slot_pool), ptr(x), int(T),
        ptr(out), ptr(topk_ids), ptr(topk_gates), ptr(miss_rows), ptr(n_miss), ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def hptr(a):
    """Host address of a numpy array or CPU tensor, or None for None."""
    if a is None:
        return None
    return a.ctypes.data if hasattr(a, "ctypes") else a.data_ptr()


def make_host_bank(fmt, n_experts, hidden, inter, tensors):
    """Bank struct over host arrays (dict with w13, w13_scale, w2, w2_scale and, for q3, w13_hi, w2_hi)."""
    f = FMT_BY_NAME[fmt] if isinstance(fmt, str) else fmt
    g = tensors.get
    return Bank(f, n_experts, hidden, inter, hptr(g("w13")), hptr(g("w13_hi")), hptr(g("w13_scale")), hptr(g("w2")),
                hptr(g("w2_hi")), hptr(g("w2_scale")))


def cpu_isa():
    return int(lib().moe_cpu_isa())


def cpu_expert_ffn(bank, x, T, k, topk_ids, topk_gates, rows, n_rows, y, n_threads=0):
    """Host call: every array is host memory (numpy or CPU tensor)."""
    _check("moe_cpu_expert_ffn", lib().moe_cpu_expert_ffn(
        ctypes.byref(bank), hptr(x), int(T), int(k), hptr(topk_ids), hptr(topk_gates), hptr(rows), int(n_rows),
        hptr(y), int(n_threads)))


def tiered_host_bytes(layer, T):
    return int(lib().moe_tiered_host_bytes(ctypes.byref(layer), int(T)))


def layer_forward_tiered(layer, layer_idx, n_layers, slot_of, slot_pool, host_bank, x, T, out, topk_ids, topk_gates,
                         miss_rows, n_miss, ws, host_ws, n_threads=0, stream=None):
    """host_ws: pinned CPU tensor of at least tiered_host_bytes(layer, T) bytes."""
    _check("moe_layer_forward_tiered", lib().moe_layer_forward_tiered(
        ctypes.byref(layer), int(layer_idx), int(n_layers), ptr(slot_of), ctypes.byref(slot_pool),
        ctypes.byref(host_bank), ptr(x), int(T), ptr(out), ptr(topk_ids), ptr(topk_gates), ptr(miss_rows),
        ptr(n_miss), ptr(ws), ws.numel() * ws.element_size(), hptr(host_ws),
        host_ws.numel() * host_ws.element_size(), int(n_threads), _stream(stream)))


def expert_usage(topk_ids, n_ids, E, counts, decay_shift=0, stream=None):
    """counts (device uint32/int32 [E]) = (counts >> decay_shift) + selections of each expert in topk_ids."""
    _check("moe_expert_usage", lib().moe_expert_usage(ptr(topk_ids), int(n_ids), int(E), ptr(counts),
                                                      int(decay_shift), _stream(stream)))


def cache_plan(counts, slot_row, layer_slots, max_moves):
    """Host call on numpy arrays: returns (move_experts, move_slots) int32 arrays."""
    import numpy as np
    counts = np.ascontiguousarray(counts, dtype=np.uint32)
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    layer_slots = np.ascontiguousarray(layer_slots, dtype=np.int32)
    me = np.zeros(max(int(max_moves), 1), dtype=np.int32)
    ms = np.zeros_like(me)
    n = np.zeros(1, dtype=np.int32)
    _check("moe_cache_plan", lib().moe_cache_plan(hptr(counts), hptr(slot_row), len(slot_row), hptr(layer_slots),
                                                  len(layer_slots), int(max_moves), hptr(me), hptr(ms), hptr(n)))
    return me[:n[0]].copy(), ms[:n[0]].copy()


def cache_refill(host_bank, slot_pool, slot_of, layer_idx, n_layers, E, move_experts, move_slots, done_event,
                 stream=None, copy_stream=None):
    """move lists: host int32 numpy arrays; done_event: a hipEvent_t handle (int)."""
    _check("moe_cache_refill", lib().moe_cache_refill(
        ctypes.byref(host_bank), ctypes.byref(slot_pool), ptr(slot_of), int(layer_idx), int(n_layers), int(E),
        hptr(move_experts), hptr(move_slots), len(move_experts), done_event, _stream(stream), copy_stream))


def cache_commit(slot_of, layer_idx, n_layers, E, n_slots, move_experts, move_slots, done_event, stream=None):
    _check("moe_cache_commit", lib().moe_cache_commit(
        ptr(slot_of), int(layer_idx), int(n_layers), int(E), int(n_slots), hptr(move_experts), hptr(move_slots),
        len(move_experts), done_event, _stream(stream)))


def time_next_launch(kernel, start_event, stop_event):
    """Arm hipEvent_t handles (ints) around the next launch of ``kernel``."""
    _check("moe_time_next_launch", lib().moe_time_next_launch(int(kernel), start_event, stop_event))


def rmsnorm_bf16(x, T, H, out, stream=None):
    _check("moe_rmsnorm_bf16", lib().moe_rmsnorm_bf16(ptr(x), int(T), int(H), ptr(out), _stream(stream)))

"""Upload host weight buffers (numpy) to device tensors and build the C structs.

Plumbing only: the buffers are copied as raw bytes; their meaning is defined by
include/moe.h and interpreted by the library's kernels.
"""
import numpy as np
import torch

from . import binding as B


def to_device(arr, device="cuda"):
    """numpy array -> device tensor with the same bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device, non_blocking=False)


class DeviceBank:
    """A bank of experts resident on the device (keeps its tensors alive)."""

    def __init__(self, fmt, n_experts, hidden, inter, arrays, device="cuda"):
        self.fmt, self.n_experts, self.hidden, self.inter = fmt, n_experts, hidden, inter
        self.tensors = {name: to_device(a, device) for name, a in arrays.items()}
        t = self.tensors
        self.struct = B.make_bank(fmt, n_experts, hidden, inter, t.get("w13"), t.get("w13_hi"), t.get("w13_scale"),
                                  t.get("w2"), t.get("w2_hi"), t.get("w2_scale"))

    def nbytes(self):
        return sum(v.numel() * v.element_size() for v in self.tensors.values())


class DeviceLayer:
    """Router weight (+ bias), routed bank and optional shared bank on the device."""

    def __init__(self, hidden, n_experts, top_k, inter, w_router, router_bias, routed, shared=None, device="cuda"):
        self.hidden, self.n_experts, self.top_k, self.inter = hidden, n_experts, top_k, inter
        self.w_router = to_device(w_router, device)
        self.router_bias = None if router_bias is None else to_device(np.asarray(router_bias, np.float32), device)
        self.routed, self.shared = routed, shared
        self.struct = B.make_layer(hidden, n_experts, top_k, inter, self.w_router, self.router_bias, routed.struct,
                                   shared.struct if shared is not None else None)

    def workspace(self, T, device="cuda"):
        """Zero-filled workspace tensor for up to T tokens."""
        n = B.workspace_bytes(self.struct, T)
        if n <= 0:
            raise ValueError("invalid layer shape")
        return torch.zeros(n, dtype=torch.uint8, device=device)

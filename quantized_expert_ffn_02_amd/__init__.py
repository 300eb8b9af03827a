"""MI355X-native quantized MoE layer: HIP kernels for gfx950 behind the C ABI in
include/moe.h, with a ctypes binding (``binding``) and device-side helpers to
upload seeded layers (``layers``)."""
from . import binding  # noqa: F401

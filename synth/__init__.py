"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side runs.

This package draws random numbers and nothing else: it holds none of the MoE
layer's arithmetic (no routing, no dequantisation, no bit layout).  Both sides
receive the same byte buffers from it and interpret them on their own.
"""
from .inputs import *  # noqa: F401,F403
from .configs import CACHE_SLOT_BUDGETS, CONFIGS, LayerShape  # noqa: F401

"""The five workloads, as shapes, formats and seeds (no arithmetic of the layer).

Shapes follow the model the pages describe: 512 experts per layer, 10 routed
plus 1 shared expert per token, hidden size 2,560, 48 layers (page "Strata Runs
125B Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "What it is"; page
"Strata: a 125B AI model on your gaming PC", model spec table).  The pages do
not state the expert intermediate size; 640 is the size that matches their
"about 700 more experts per extra GB of VRAM" at 2.5 bits per weight (page
"Strata Runs 125B ...", section "How a 125B model fits in 12 GB").
Prompt chunks of up to 8,192 tokens and MTP verify batches of 1 + 3 tokens come
from page "Strata Runs a 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU
at up to 93 Tokens per Second" (speculative decoding and chunked reading).
"""
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class LayerShape:
    hidden: int = 2560
    n_experts: int = 512
    top_k: int = 10
    inter: int = 640
    shared: bool = True
    fmt: str = "q2"            # "bf16" | "q2" | "q3"
    zipf: Optional[float] = None  # Zipf exponent of the router-bias popularity, None = no bias


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    shape: LayerShape
    tokens: Tuple[int, ...]
    layers: int = 1
    slots: int = 0             # expert-cache slots (cache workload only)
    slots_per_layer: int = 0


CONFIGS = {
    # Tiny unquantised layer: 16 experts, top-4 + shared, bf16 weights N(0, 0.02), 4 tokens.
    "tiny": Workload("tiny", 1, LayerShape(2560, 16, 4, 640, True, "bf16", None), (4,)),
    # One real-shape 2-bit layer, decode: 1 token and 1 + 3 MTP verify tokens.
    "decode": Workload("decode", 2, LayerShape(2560, 512, 10, 640, True, "q2", None), (1, 4)),
    # Same layer, one 8,192-token prefill chunk with Zipf(1.1)-skewed routing.
    "prefill": Workload("prefill", 3, LayerShape(2560, 512, 10, 640, True, "q2", 1.1), (8192,)),
    # 48 independent 2-bit layers with residual adds, batch 1 and 32 x 4 = 128 verify tokens.
    "stack": Workload("stack", 4, LayerShape(2560, 512, 10, 640, True, "q2", 1.1), (1, 128), layers=48),
    # 3-bit layer with a 3,072-slot expert cache (top 64 experts of each of 48 layers), 64 tokens.
    "cache": Workload("cache", 5, LayerShape(2560, 512, 10, 640, True, "q3", 1.1), (64,), layers=48,
                      slots=3072, slots_per_layer=64),
    # The pruned "Coder" build: 256 of 512 experts kept per layer, still top-10 + shared (page "Strata Runs 125B
    # Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "The Coder build: half the experts, most of the skill").
    "coder": Workload("coder", 6, LayerShape(2560, 256, 10, 640, True, "q2", None), (1, 4, 64)),
}

# Expert-cache sizes the pages report: 1,589 cached experts at 262K context with the KV cache on the GPU, 3,872
# once most of it moves to RAM (page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "How a
# 125B model fits in 12 GB"); 3,072 is the cache workload's own size.
CACHE_SLOT_BUDGETS = (1589, 3072, 3872)

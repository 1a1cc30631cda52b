"""Workload sizes as the pages state them.

Source: guide ch. 1 "The problem, the judge and the speed of light",
§1.1 (layer table: N x K, dtypes, the unpooler's 1024-row slice at <= 8 tokens)
and §1.2 (the six loads and the awkward token counts checked for correctness).
"""

# Layer order is fixed: it is also the integer layer id used at the C ABI.
LAYERS = ("qkv_gate", "o", "pooler", "unpooler", "router")
LAYER_ID = {name: i for i, name in enumerate(LAYERS)}
ROUTER = "router"

# (N output features, K input features), guide ch. 1 §1.1 layer table.
SHAPES = {
    "qkv_gate": (2304, 8192),
    "o": (8192, 1024),
    "pooler": (4096, 8192),
    "unpooler": (8192, 4096),
    "router": (256, 8192),
}

# Token count m of each load, guide ch. 1 §1.2 load table.
LOADS = {
    "decode-1": 1,
    "decode-16": 16,
    "decode-32": 32,
    "verify-1": 8,
    "verify-16": 128,
    "verify-32": 256,
}

# Correctness-only token counts, guide ch. 1 §1.2 (the list after the load table).
AWKWARD_M = (5, 7, 9, 33, 130, 512, 1000)


def weight_dtype(layer):
    """Storage type of W: FP32 for the router, BF16 otherwise (guide ch. 1 §1.1)."""
    return "f32" if layer == ROUTER else "bf16"


def out_dtype(layer):
    """Storage type of out: FP32 for the router, BF16 otherwise (guide ch. 1 §1.1)."""
    return "f32" if layer == ROUTER else "bf16"

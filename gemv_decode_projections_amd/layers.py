"""Layer table of the GPU library's Python side.

The five projections and their shapes (guide ch. 1 "The problem, the judge and
the speed of light", §1.1). The C library holds the same table and reports it
through proj_layer_dims; tests check the two agree.
"""

LAYERS = ("qkv_gate", "o", "pooler", "unpooler", "router")
LAYER_ID = {name: i for i, name in enumerate(LAYERS)}

# name -> (N, K, weight bytes per element, out bytes per element)
DIMS = {
    "qkv_gate": (2304, 8192, 2, 2),
    "o": (8192, 1024, 2, 2),
    "pooler": (4096, 8192, 2, 2),
    "unpooler": (8192, 4096, 2, 2),
    "router": (256, 8192, 4, 4),
}

# At <= 8 tokens only the unpooler's first 1024 rows are computed (§1.1).
UNPOOLER_SLICE_M = 8
UNPOOLER_SLICE_ROWS = 1024


def layer_id(layer):
    if isinstance(layer, int):
        if not 0 <= layer < len(LAYERS):
            raise ValueError("unknown layer id %d" % layer)
        return layer
    return LAYER_ID[layer]


def layer_name(layer):
    return LAYERS[layer_id(layer)]


def n_eff(layer, m):
    name = layer_name(layer)
    n = DIMS[name][0]
    if name == "unpooler" and m <= UNPOOLER_SLICE_M:
        return UNPOOLER_SLICE_ROWS
    return n

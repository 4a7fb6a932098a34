"""ctypes declarations of libmoe_mi355x.so (include/moe_mi355x.h)."""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_LIMIT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

MOE_IDX_I32 = 0
MOE_IDX_I64 = 1
MOE_W_BF16 = 0
MOE_W_FP8_E4M3 = 1
MOE_W_BF16_TILED = 2
MOE_W_FP8_E4M3_TILED = 3
MOE_W_FP8_E4M3_ROWS = 4
MOE_W_FP8_E4M3_ROWS_TILED = 5
MOE_W_MXFP4 = 6
MOE_W_MXFP4_TILED = 7
MOE_MAX_EXPERTS = 1024
MOE_ROUTER_MAX_TOP_K = 64
MOE_FUSED_ALIGN_MAX_SLOTS = 2048
MOE_FUSED_LAYER_MAX_SLOTS = 256
MOE_LAYER_PATH_AUTO = 0
MOE_LAYER_PATH_STEPS = 1
MOE_LAYER_PATH_SINGLE_PASS = 2
MOE_LAYER_PATH_NARROW = 3
MOE_NARROW_LAYER_MAX_SLOTS = 32
MOE_NARROW_AUTO_SLOTS = 24
MOE_LAYER_WORKSPACE_REGIONS = 14
MOE_NOALLOC_WORKSPACE_BYTES = 64 << 20

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t

TABLE_FIELDS = ("sorted_token_ids", "block_expert_ids", "expert_offsets", "expert_counts",
                "token_to_perm", "active_experts", "active_count", "total")


class MoeAlignTables(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in TABLE_FIELDS]


class MoeWeight(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p)]


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [
        ("M", c_int64), ("H", c_int32), ("I", c_int32), ("S", c_int32), ("E", c_int32),
        ("top_k", c_int32), ("BS", c_int32), ("wdt", c_int), ("idt", c_int),
        ("gate", MoeWeight), ("up", MoeWeight), ("down", MoeWeight),
        ("sh_gate", MoeWeight), ("sh_up", MoeWeight), ("sh_down", MoeWeight),
        ("sh_expert_gate", c_void_p), ("path", c_int),
    ]


P = ctypes.POINTER

# every symbol the header declares, with its C signature
SIGNATURES = {
    "moe_align_max_total": (c_int64, [c_int64, c_int32, c_int32]),
    "moe_active_cap": (c_int32, [c_int64, c_int32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (c_int32, []),
    "moe_align": (c_int, [c_void_p, c_int, c_int64, c_int32, c_int32, c_int32, P(MoeAlignTables), c_void_p]),
    "moe_align_workspace_bytes": (c_size_t, [c_int64, c_int32, c_int32]),
    "moe_align_ws": (c_int, [c_void_p, c_int, c_int64, c_int32, c_int32, c_int32, P(MoeAlignTables), c_void_p,
                             c_size_t, c_void_p]),
    "moe_grouped_gate_up_silu": (c_int, [c_void_p, c_int, P(MoeWeight), P(MoeWeight), P(MoeAlignTables),
                                         c_void_p, P(MoeWeight), P(MoeWeight), c_void_p, c_int64, c_int32,
                                         c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "moe_align_gate_up_silu": (c_int, [c_void_p, c_int, c_void_p, c_int, P(MoeWeight), P(MoeWeight),
                                       P(MoeAlignTables), c_void_p, P(MoeWeight), P(MoeWeight), c_void_p, c_int64,
                                       c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "moe_grouped_down": (c_int, [c_void_p, c_int, P(MoeWeight), P(MoeAlignTables), c_void_p, P(MoeWeight),
                                 c_void_p, c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_void_p]),
    "moe_blend": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                          c_int32, c_void_p]),
    "moe_layer_workspace_bytes": (c_size_t, [P(MoeLayerDesc)]),
    "moe_layer_forward": (c_int, [P(MoeLayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                  c_void_p]),
    "moe_layer_workspace_layout": (c_int, [P(MoeLayerDesc), P(c_size_t)]),
    "moe_layer_path": (c_int, [P(MoeLayerDesc)]),
    "moe_layer_partials": (c_int, [P(MoeLayerDesc), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_layer_blend_partials": (c_int, [P(MoeLayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_size_t, c_void_p]),
    "moe_tiled_weight_bytes": (c_size_t, [c_int, c_int64, c_int32, c_int32]),
    "moe_stream_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]),
    "moe_router_topk": (c_int, [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int,
                                c_void_p, c_void_p]),
    "moe_tile_weights": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int32, c_int32, c_void_p]),
    "moe_layer_forward_noalloc": (c_int, [P(MoeLayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
}

_LIB = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (no fallback: a missing build is an error)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m mixture_experts_routing_align_amd.build, or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB

"""Loads libhydra.so and declares the C signatures of include/hydra.h."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# HYDRA_LIB selects another build of the same sources (the sanitized one of
# build.py --sanitize, for host-side checks)
LIB_PATH = os.environ.get("HYDRA_LIB") or os.path.join(_HERE, "libhydra.so")

c_int, c_float, c_size, c_void = C.c_int, C.c_float, C.c_size_t, C.c_void_p
i32p = C.POINTER(C.c_int32)

# name -> (restype, argtypes), in the order of include/hydra.h
SIGNATURES = {
    "hydra_status_string": (C.c_char_p, [c_int]),
    "hydra_last_error": (C.c_char_p, []),
    "hydra_abi_version": (c_int, []),
    "hydra_plan_cartesian": (c_int, [i32p, c_int, c_int, i32p, i32p, i32p]),
    "hydra_plan_sparse": (c_int, [i32p, c_int, c_int, c_int, i32p, i32p, i32p]),
    "hydra_plan_rows": (c_int, [c_int, i32p, i32p, i32p, c_int, i32p, i32p, i32p, i32p, i32p]),
    "hydra_draft_heads_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, i32p]),
    "hydra_draft_heads": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void,
                                  C.POINTER(c_void), c_int,
                                  C.POINTER(c_void), C.POINTER(c_void), C.POINTER(c_void), c_int, c_int,
                                  c_void, c_void, c_void, c_int, c_void, i32p, i32p, i32p, c_void, c_void,
                                  c_void, c_void, c_void, c_void, c_size, c_void]),
    "hydra_draft_heads_sketch_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, i32p]),
    "hydra_draft_heads_sketch": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_int]
                                 + [C.POINTER(c_void)] * 7
                                 + [c_float, c_int, c_int, c_void, c_void, c_void, c_int, c_void, i32p, i32p, i32p,
                                    c_void, c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
    "hydra_draft_heads_attn_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, i32p]),
    "hydra_draft_heads_attn": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_void,
                                       c_int, C.POINTER(c_void), C.POINTER(c_void), C.POINTER(c_void), c_int, c_int,
                                       c_void, c_void, c_void, c_int, c_void, i32p, i32p, i32p, c_void, c_void,
                                       c_void, c_void, c_void, c_void, c_size, c_void]),
    "hydra_fold_embedding": (c_int, [c_int, c_int, c_int, c_void, c_void, c_void, c_void]),
    "hydra_vocab_projection_workspace_size": (c_size, [c_int, c_int, c_int]),
    "hydra_vocab_projection": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_size,
                                       c_void]),
    "hydra_packed_weight_size": (c_size, [c_int, c_int]),
    "hydra_pack_weight": (c_int, [c_int, c_int, c_void, c_void, c_void]),
    "hydra_vocab_topk": (c_int, [c_int, c_int, c_int, c_void, c_void, c_size, c_void, c_void, c_void, c_void]),
    "tree_build_workspace_size": (c_size, [c_int, c_int, c_int]),
    "tree_build": (c_int, [c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_void, c_void, c_int,
                           c_void, c_void, c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
    "tree_rope": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_float, c_void]),
    "tree_rope_qk": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_void,
                             c_void, c_float, c_void]),
    "tree_attention_verify_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "tree_attention_verify": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void, c_void,
                                      c_void, c_void, c_void, c_int, c_int, c_void, c_int, c_void, c_int,
                                      c_void, c_void, c_int, c_void, c_void, c_void, c_size, c_void]),
    "tree_decoder_layer_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "tree_decoder_layer": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void,
                                   c_void, c_void, c_void, c_void, c_float, c_float, c_void, c_void, c_int, c_int,
                                   c_void, c_int, c_void, c_int, c_void, c_void, c_int, c_void, c_void, c_void,
                                   c_void, c_size, c_void]),
    "tree_verify_layers_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "tree_verify_layers": (c_int, [c_int] * 10 + [c_void] * 9 + [c_float, c_float, c_void, c_void, c_int, c_int,
                                                                c_void, c_int, c_void, c_int, c_void, c_void, c_int,
                                                                c_void, c_void, c_void, c_void, c_size, c_void]),
    "tree_accept_workspace_size": (c_size, [c_int, c_int, c_int, c_int]),
    "tree_accept": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_float, c_float,
                            c_float, c_void, c_void, c_void, c_void, c_int, c_void, c_void, c_void, c_void, c_void,
                            c_void, c_void, c_size, c_void]),
    "tree_accept_noalloc": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_float,
                                    c_float, c_float, c_void, c_void, c_void, c_void, c_int, c_void, c_void, c_void,
                                    c_void, c_void, c_void, c_void]),
    "tree_commit": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void,
                            c_int, c_int, c_void, c_int, c_void, c_void, c_void, c_void, c_int, c_void, c_void,
                            c_void, c_void, c_void]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_hydra_amd.build` "
                "(there is no fallback path)")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib

"""ctypes view of libduo.so (the C ABI in include/duo.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI. If the library has not been built this module
raises at import time; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libduo.so")

DUO_OK, DUO_ERR_INVALID_ARG, DUO_ERR_UNSUPPORTED, DUO_ERR_LAYOUT, DUO_ERR_CAPACITY, DUO_ERR_HIP = range(6)
DUO_BF16, DUO_FP16, DUO_INT4_G32 = 0, 1, 2
DUO_GRAD_SCRATCH_PARTIALS = 65536  # slots of duo_mixed_alpha_grad_noalloc's device array
DTYPES = {"bf16": DUO_BF16, "fp16": DUO_FP16, "int4": DUO_INT4_G32}


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32),
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("n_retrieval_kv_heads", c_int32),
        ("sink", c_int32),
        ("recent", c_int32),
        ("retrieval_capacity", c_int64),
        ("kv_dtype", c_int),
        ("retrieval_dtype", c_int),
        ("softmax_scale", c_float),
    ]


class Layout(ctypes.Structure):
    _fields_ = [(name, c_size_t) for name in (
        "retrieval_bytes", "streaming_bytes", "workspace_bytes", "k_offset", "v_offset",
        "k_sz_offset", "v_sz_offset", "ring_k_offset", "ring_v_offset")]


class DuoError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kv_cache_compression_duo_amd.build` "
            "(there is no fallback path)")
    # torch's HIP runtime has to be in the process before the library is opened: the
    # library's libamdhip64 dependency then resolves to that same runtime, which owns the
    # device memory and streams torch hands over. Opened first, the library would pull in
    # a second HIP runtime, and that second copy finds no device next to torch's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "duo_layer_layout": (c_int, [POINTER(LayerDesc), POINTER(Layout)]),
        "duo_layer_init": (c_int, [POINTER(c_void_p), POINTER(LayerDesc), c_void_p, c_void_p,
                                   c_void_p, c_int64, c_void_p]),
        "duo_layer_init_ragged": (c_int, [POINTER(c_void_p), POINTER(LayerDesc), c_void_p,
                                          c_void_p, c_void_p, POINTER(c_int64), c_void_p]),
        "duo_layer_destroy": (c_int, [c_void_p]),
        "duo_layer_tokens": (c_int64, [c_void_p]),
        "duo_layer_sequence_tokens": (c_int64, [c_void_p, c_int32]),
        "duo_append_kv_seq": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p]),
        "duo_prefill_chunk_seq": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                          c_void_p, c_void_p]),
        "duo_append_kv": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
        "duo_prefill_chunk": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                      c_void_p]),
        "duo_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "duo_mixed_forward": (c_int, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int32, c_void_p, c_void_p]),
        "duo_mixed_forward_block": (c_int, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
        "duo_mixed_alpha_grad_block": (c_int, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_void_p, c_float, c_int32, c_int32,
                                               c_void_p, c_void_p, c_size_t, c_void_p]),
        "duo_mixed_alpha_grad_noalloc": (c_int, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_float, c_int32, c_int32,
                                                 c_void_p, c_void_p]),
        "duo_mixed_alpha_grad_workspace": (c_size_t, [POINTER(LayerDesc), c_int32]),
        "duo_mixed_alpha_grad": (c_int, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_float, c_int32, c_void_p,
                                         c_void_p, c_size_t, c_void_p]),
        "duo_head_permutation": (c_int, [POINTER(c_uint8), c_int32, POINTER(c_int32),
                                         POINTER(c_int32)]),
        "duo_binarize_gates": (c_int, [POINTER(c_float), c_int32, ctypes.c_double,
                                       POINTER(c_uint8)]),
        "duo_reorder_head_rows": (c_int, [c_void_p, c_void_p, POINTER(c_int32), c_int32, c_int64,
                                          c_int64]),
        "duo_ring_slot": (c_int32, [c_int64, c_int32, c_int32]),
        "duo_status_string": (c_char_p, [c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.duo_status_string(status).decode()


def check(status: int, what: str):
    if status != DUO_OK:
        raise DuoError(status, what)


def make_desc(*, batch=1, n_q_heads, n_kv_heads, head_dim, n_retrieval_kv_heads, sink=16,
              recent=64, capacity=0, kv_dtype="bf16", retrieval_dtype=None,
              softmax_scale=1.0) -> LayerDesc:
    rd = kv_dtype if retrieval_dtype is None else retrieval_dtype
    return LayerDesc(batch, n_q_heads, n_kv_heads, head_dim, n_retrieval_kv_heads, sink, recent,
                     capacity, DTYPES[kv_dtype], DTYPES[rd], softmax_scale)


def layout(desc: LayerDesc) -> Layout:
    out = Layout()
    check(lib.duo_layer_layout(byref(desc), byref(out)), "duo_layer_layout")
    return out

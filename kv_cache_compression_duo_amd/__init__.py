"""DuoAttention head-split attention for AMD Instinct MI355X (gfx950).

Retrieval heads: full causal attention over a full KV cache (bf16/fp16 or
4-bit groups). Streaming heads: Lambda-masked attention over a sink + recent
ring. Chunked prefill, decode and the alpha-blended identification forward
run in hand-written HIP kernels behind the C ABI of include/duo.h; this
package is the thin ctypes binding (torch supplies device memory and streams).
"""
from ._lib import DuoError, LIB_PATH, status_string
from .api import (DuoLayer, mixed_forward, mixed_alpha_grad, mixed_alpha_grad_noalloc,
                  binarize_gates, reorder_head_rows, head_permutation, ring_slot)

__all__ = ["DuoError", "LIB_PATH", "status_string", "DuoLayer", "mixed_forward", "mixed_alpha_grad",
           "mixed_alpha_grad_noalloc",
           "binarize_gates", "reorder_head_rows",
           "head_permutation", "ring_slot"]

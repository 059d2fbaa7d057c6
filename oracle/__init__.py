"""CPU oracle for the DuoAttention hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 NumPy statement of what the hot path
computes. Only the test-suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product library never
calls it, and it shares no code with the HIP path: no kernels, headers,
helpers, tables or pre/post-processing. The only module both sides use is the
seeded input generator ``duo_synth`` (random numbers and rounding to the
storage dtype, nothing of the method).

Sources (cited by page and section):
  * xllm-io review -- "DuoAttention: Efficient Long-Context LLM Inference with
    Retrieval and Streaming Heads", Chinese paper review on xllm-io.github.io
    (sections 一 ... 八). The only page that prints the formulas.
  * paperlayer summary -- the same title, AI summary of arXiv 2410.10819v1 on
    paperlayer.ai (sections 1-5, A.1-A.5).
  * scime atlas summary -- the same title, AI summary on atlas.scime.ai.

Readings where the pages are silent or garbled are stated where they are
used. Every function here is pinned by tests in
``tests/test_oracle_*.py`` against brute force, a library routine, closed
forms or the pages' invariants; the one exception is marked
"parity unpinned" in its docstring (none at present).
"""
from .attention import (allowed_mask, masked_attention, layer_attention,
                        mixed_attention, full_attention, streaming_attention)
from .cache import ring_slot, ring_positions_after, OracleLayer
from .int4 import quantize_int4_g32, dequantize_int4_g32, pack_nibbles, unpack_nibbles
from .routing import head_permutation, apply_head_permutation, invert_permutation
from .gates import mixed_alpha_grad, binarize_gates, reorder_head_rows

__all__ = [
    "allowed_mask", "masked_attention", "layer_attention", "mixed_attention",
    "full_attention", "streaming_attention",
    "ring_slot", "ring_positions_after", "OracleLayer",
    "quantize_int4_g32", "dequantize_int4_g32", "pack_nibbles", "unpack_nibbles",
    "head_permutation", "apply_head_permutation", "invert_permutation",
    "mixed_alpha_grad", "binarize_gates", "reorder_head_rows",
]

"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. The HIP library and its Python binding never do.
"""

from .vqv_ref import (GROUP, accept_walk_ref, argmax_ref, decode_act, decode_f16,
                      dequantize, margin_ref, qgemm_ref, qgemm_swiglu_ref, silu_ref, swiglu_ref,
                      unpack_codes, verify_ref)

__all__ = ["GROUP", "accept_walk_ref", "argmax_ref", "decode_act", "decode_f16",
           "dequantize", "margin_ref", "qgemm_ref", "qgemm_swiglu_ref", "silu_ref", "swiglu_ref",
           "unpack_codes", "verify_ref"]

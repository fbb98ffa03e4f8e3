"""CPU oracle for the fp8 query of the fp8 decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it.

With an fp8 KV cache the pages cast the query to float8_e4m3fn, with a query
scale of 1, before their fp8 decode kernel: ``TRTLLMMLABackend.forward_decode``
on "tokenspeed trtllm_mla.py" (the cast of q) and ``forward_decode`` on
"sglang trtllm_mla_backend.py" (``mla_quantize_and_rope_for_fp8``, which turns
the rope part first); ``_compute_decode_bmm1_scale`` on the latter fixes
q_scale = 1.  The decode then attends with the codes' values.

What this computes: each query element, a bf16 value (after the rotation,
when one applies, rounded to bf16 as ``rope.rotate_query`` returns it),
becomes its OCP e4m3fn code (``kv_append.e4m3fn_encode``: nearest value, ties
to the even code, saturated at +-448, NaN kept), and the code's value is
returned as a bf16 bit pattern.  Every e4m3fn value is a bf16 value (at most
four significant bits, exponents -9 .. 8), so the pattern is exact and the
decode oracle runs on it unchanged.

Readings (where the pages leave it open): finite values beyond +-448 saturate
(torch's own cast, the pages' ``q.to(torch.float8_e4m3fn)``, gives NaN there);
the rotation is rounded to bf16 before the cast.

Pinned by ``tests/test_oracle_query_fp8.py``: torch's float8 cast over every
in-range bf16 pattern, closed forms of the saturation and the ties.
"""
from __future__ import annotations

import numpy as np

from .kv_append import e4m3fn_encode, e4m3fn_value, E4M3FN_NAN


def _code_values_f32() -> np.ndarray:
    """float32 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    v = np.array([np.nan if (c & 0x7F) == E4M3FN_NAN else e4m3fn_value(c) for c in range(256)], dtype=np.float64)
    return v.astype(np.float32)


_VALUES = _code_values_f32()


def quantize_query(q_bits) -> np.ndarray:
    """bf16 bit patterns (any shape) -> bf16 bit patterns of the e4m3fn values
    of their codes."""
    bits = np.asarray(q_bits, dtype=np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    v = _VALUES[e4m3fn_encode(x)]
    out = (v.view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), out).reshape(bits.shape)

"""CPU oracle for the KV-cache append -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it.

What it computes is the cache write that precedes every decode on the pages:
``set_mla_kv_buffer(layer, out_cache_loc, k_nope, k_rope)`` in
``TRTLLMMLABackend.forward_decode`` ("sglang trtllm_mla_backend.py") and in
``TRTLLMMLABackend.forward_decode`` ("tokenspeed trtllm_mla.py").  Row i,
the 512-wide latent ``k_nope[i]`` followed by the 64-wide rope key
``k_rope[i]``, is stored in the flat slot ``out_cache_loc[i]`` of the pool,
that is in page ``loc // page_size``, slot ``loc % page_size`` (the same
token -> (page, slot) map the decode reads through).  A bf16 pool stores the
bf16 bits unchanged.  An fp8 pool stores the OCP float8_e4m3fn code of
``x / k_scale`` (the per-tensor scale convention of ``scaled_fp8_quant`` in
``_quantize_fp8_qkv``, "sglang trtllm_mla_backend.py"), computed in float32,
saturated to +-448 (the largest finite e4m3fn value), rounded to nearest with
ties to even; a NaN stores 0x7F.  Locations outside [0, num_pages*page_size)
are skipped.

The encoder is written from the format's definition, with no bit tricks:
every non-negative finite code's value is listed from (exponent, mantissa),
and a magnitude takes the nearest listed value, the code with an even
mantissa on a tie.  ``tests/test_oracle_append.py`` pins it against torch's
own float8 cast and the closed forms of the format.
"""
from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0
E4M3FN_NAN = 0x7F
LATENT = 512
ROPE = 64
ROW = LATENT + ROPE


def e4m3fn_value(code: int) -> float:
    """Value of a non-NaN e4m3fn code: sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 holds the subnormals m/8 * 2^-6."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the 127 non-negative finite codes 0x00 .. 0x7E, in increasing value
_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)
_POS_VALUES = np.array([e4m3fn_value(int(c)) for c in _POS_CODES], dtype=np.float64)


def e4m3fn_encode(x) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8): saturate to +-448, round to the
    nearest value, ties to the even code; NaN -> 0x7F; the sign of -0 kept."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    flat = x.reshape(-1)
    nan = np.isnan(flat)
    neg = np.signbit(flat)
    a = np.minimum(np.abs(np.where(nan, 0.0, flat)), E4M3FN_MAX)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 16
    for s in range(0, flat.size, step):
        d = np.abs(a[s:s + step, None] - _POS_VALUES[None, :])
        idx = np.argmin(d, axis=1)                       # the first (smaller) of two equally near values
        nxt = np.minimum(idx + 1, len(_POS_VALUES) - 1)
        rows = np.arange(idx.size)
        tie = (nxt != idx) & (d[rows, nxt] == d[rows, idx])
        idx = np.where(tie & (_POS_CODES[idx] % 2 == 1), nxt, idx)   # tie: the even code
        out[s:s + step] = _POS_CODES[idx]
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    out[nan] = E4M3FN_NAN
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: the bits are the top half of a float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_rows(rows_bf16_bits, k_scale: float) -> np.ndarray:
    """[T, 576] bf16 bits -> [T, 576] e4m3fn codes of x / k_scale (float32 division)."""
    x = bf16_bits_to_f32(rows_bf16_bits)
    with np.errstate(over="ignore", invalid="ignore"):
        q = x / np.float32(k_scale)
    return e4m3fn_encode(q)


def kv_append(pool: np.ndarray, k_nope_bits: np.ndarray, k_rope_bits: np.ndarray, out_cache_loc: np.ndarray,
              k_scale: float = 1.0) -> np.ndarray:
    """A copy of ``pool`` ([N, P, 576], uint16 bf16 bits or uint8 e4m3fn codes)
    with row i = [k_nope[i] | k_rope[i]] (bf16 bits, [T, 512] and [T, 64])
    stored at flat slot out_cache_loc[i]; out-of-range locations are skipped."""
    pool = np.array(pool, copy=True)
    N, P, D = pool.shape
    assert D == ROW
    nope = np.asarray(k_nope_bits, dtype=np.uint16)
    rope = np.asarray(k_rope_bits, dtype=np.uint16)
    T = nope.shape[0]
    assert nope.shape == (T, LATENT) and rope.shape == (T, ROPE)
    rows = np.concatenate([nope, rope], axis=1)
    if pool.dtype == np.uint8:
        rows = quantize_rows(rows, k_scale)
    loc = np.asarray(out_cache_loc, dtype=np.int64)
    for i in range(T):
        s = int(loc[i])
        if 0 <= s < N * P:
            pool[s // P, s % P, :] = rows[i]
    return pool

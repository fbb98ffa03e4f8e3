"""CPU oracle for rotary position embedding of the rope parts -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it.

The pages hand the decode the query's rope part and the new key's rope part
together with the token positions, a cos/sin cache and an ``is_neox`` flag
(``forward_decode`` of ``TRTLLMMLABackend`` on "sglang trtllm_mla_backend.py"
and "tokenspeed trtllm_mla.py", which pass them to the vendor rope-and-quantise
kernel).  The rotation is the standard rotary embedding: the 64 rope
dimensions form 32 pairs (x1, x2), pair i turned by the angle of frequency i
at the token's position, whose cosine and sine are row ``pos`` of the cache
(cos in columns 0..31, sin in 32..63):

    y1 = x1 cos - x2 sin,   y2 = x2 cos + x1 sin

With ``is_neox`` the pairs are (i, i + 32) (the rotate-half layout), otherwise
(2i, 2i + 1) (interleaved).  Precision, as the GPU does it: the bf16 inputs
widened to float32, each product and the difference or sum rounded to float32
(no fused multiply-add), the result rounded to bf16 with ties to even.
"""
from __future__ import annotations

import numpy as np

ROPE = 64
HALF = 32


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _f32_to_bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r)


def pair_index(is_neox: bool):
    """(first, second) element index of each of the 32 rotation pairs."""
    i = np.arange(HALF)
    return (i, i + HALF) if is_neox else (2 * i, 2 * i + 1)


def rotate(rope_bits: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray, is_neox: bool) -> np.ndarray:
    """rope_bits [..., 64] bf16 bits, positions broadcastable to rope_bits.shape[:-1]
    (int), cos_sin_cache float32 [max_pos, 64] -> rotated bf16 bits [..., 64]."""
    x = _bf16_to_f32(rope_bits)
    pos = np.broadcast_to(np.asarray(positions, dtype=np.int64), x.shape[:-1])
    cs = np.asarray(cos_sin_cache, dtype=np.float32)[pos]            # [..., 64]
    cos, sin = cs[..., :HALF], cs[..., HALF:]
    a, b = pair_index(is_neox)
    x1, x2 = x[..., a], x[..., b]
    y = np.empty_like(x)
    with np.errstate(over="ignore", invalid="ignore"):
        y[..., a] = (x1 * cos).astype(np.float32) - (x2 * sin).astype(np.float32)
        y[..., b] = (x2 * cos).astype(np.float32) + (x1 * sin).astype(np.float32)
    return _f32_to_bf16(y)


def rotate_query(q_bits: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray, is_neox: bool) -> np.ndarray:
    """q_bits [B, q_len, H, 576] bf16 bits, positions [B, q_len]: a copy with
    the rope part (dims 512..575) of every row rotated at its token's position."""
    out = np.array(q_bits, copy=True)
    out[..., 512:] = rotate(q_bits[..., 512:], np.asarray(positions)[..., None], cos_sin_cache, is_neox)
    return out

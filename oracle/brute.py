"""Dense brute-force MLA decode in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

An independent second implementation used to pin the C oracle on small
inputs.  It shares nothing with ``oracle.c``: it decodes the stored codes
with numpy bit operations, gathers every request's rows with one fancy index
(token -> (page, slot)), and computes dense softmax attention with library
primitives (einsum, logsumexp), masking the causal future with a
bottom-right aligned triangle:

    S = scale * Q K^T,   S[j, t] = -inf for t >= L - q_len + 1 + j
    lse = logsumexp_t S,  O = exp(S - lse) K[:, :512]

(the decode call of "sglang trtllm_mla_backend.py", _run_decode_kernel,
and the causal multi-token call of "tokenspeed flashmla.py",
FlashMLABackend.forward_extend).
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    v = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, v)


def decode(inp):
    """out [B, q_len, H, 512], lse [B, q_len, H] in float64."""
    B, ql, H, D = inp.q.shape
    P = inp.page_size
    out = np.zeros((B, ql, H, 512))
    lse = np.full((B, ql, H), -np.inf)
    for b in range(B):
        L = max(int(inp.seq_lens[b]), 0)
        t = np.arange(L)
        stored = inp.pool[inp.block_table[b, t // P], t % P] if L else inp.pool[:0, 0]
        if inp.kv_fp8:
            K = e4m3fn_codes_to_f64(stored) * inp.k_scale
        else:
            K = bf16_bits_to_f64(stored)
        Q = bf16_bits_to_f64(inp.q[b])                     # [ql, H, 576]
        S = inp.softmax_scale * np.einsum("jhd,td->jht", Q, K)
        vis = L - ql + 1 + np.arange(ql)                   # visible tokens per query token
        mask = t[None, :] < vis[:, None]                   # [ql, L]
        S = np.where(mask[:, None, :], S, -np.inf)
        with np.errstate(invalid="ignore"):
            lz = logsumexp(S, axis=-1) if L else np.full((ql, H), -np.inf)
            Pm = np.where(mask[:, None, :], np.exp(S - lz[..., None]), 0.0)
        out[b] = np.einsum("jht,tc->jhc", Pm, K[:, :512]) if L else 0.0
        lse[b] = lz
    return out, lse

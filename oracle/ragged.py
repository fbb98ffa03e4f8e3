"""CPU oracle for the ragged multi-token decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it.

A ragged batch gives request b its own number q_b of query tokens, packed
without padding at rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (the
draft-extend metadata of TRTLLMMLABackend.init_forward_metadata on
"tokenspeed trtllm_mla.py", which builds cu_seqlens_q from the per-request
extend lengths; the pages pad every request to the longest and unpad the
output afterwards).  Seq_lens count each request's q_b new tokens, so the
padded call's bottom-right alignment reads, per request,
vis(j) = L_b - q_b + 1 + j.  Requests are independent: the ragged decode is
one uniform decode per request with q_len = q_b, and that is exactly how it
is computed here, through the pinned fp64 C oracle (or the dense numpy
brute force) on a one-request view of the batch.
"""
from __future__ import annotations

import types

import numpy as np

from . import brute as _brute


def request_view(rg, b: int):
    """Request b of a ragged batch as a one-request uniform input (q_len = q_b)."""
    base = rg.base
    s, e = int(rg.qo_indptr[b]), int(rg.qo_indptr[b + 1])
    q = rg.q[s:e][None]                                   # [1, q_b, H, 576]
    v = types.SimpleNamespace(q=np.ascontiguousarray(q), pool=base.pool,
                              block_table=np.ascontiguousarray(base.block_table[b:b + 1]),
                              seq_lens=np.ascontiguousarray(base.seq_lens[b:b + 1]),
                              softmax_scale=base.softmax_scale, k_scale=base.k_scale, workload=base.workload)
    v.batch, v.q_len, v.heads = 1, e - s, q.shape[2]
    v.page_size, v.num_pages = base.page_size, base.num_pages
    v.kv_fp8 = base.kv_fp8
    v.max_seq_len = int(v.seq_lens.max())
    return v


def decode(orc, rg, dense: bool = False):
    """out [T, H, 512] and lse [T, H] (float64) of the packed query rows; orc is
    an oracle.Oracle, or dense=True for the numpy brute force."""
    T, H, _ = rg.q.shape
    out = np.zeros((T, H, 512), dtype=np.float64)
    lse = np.zeros((T, H), dtype=np.float64)
    for b in range(rg.base.batch):
        s, e = int(rg.qo_indptr[b]), int(rg.qo_indptr[b + 1])
        if e == s:
            continue
        v = request_view(rg, b)
        o, l = _brute.decode(v) if dense else orc.decode(v)
        out[s:e] = o[0]
        lse[s:e] = l[0]
    return out, lse


def decode_rows(orc, rg, sel):
    """Selected packed rows (token, h): out [n, 512], lse [n]."""
    out = np.zeros((len(sel), 512), dtype=np.float64)
    lse = np.zeros(len(sel), dtype=np.float64)
    tok_req = np.searchsorted(rg.qo_indptr, np.arange(rg.total_q), side="right") - 1
    by_req = {}
    for i, (t, h) in enumerate(sel):
        b = int(tok_req[t])
        by_req.setdefault(b, []).append((i, t - int(rg.qo_indptr[b]), h))
    for b, items in by_req.items():
        v = request_view(rg, b)
        o, l = orc.decode_rows(v, [(0, j, h) for _, j, h in items])
        for k, (i, _, _) in enumerate(items):
            out[i], lse[i] = o[k], l[k]
    return out, lse

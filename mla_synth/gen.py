"""Seeded synthetic inputs for batched paged MLA decode.

This module only produces input bytes: sequence lengths, a scattered block
table over a page pool, the absorbed query rows and the latent KV rows, in
the storage formats the decode consumes (bf16 bit patterns, or OCP
float8_e4m3fn codes).  It holds none of the attention arithmetic, so both the
CPU oracle and the GPU path can take their inputs from it.

Shapes follow the decode call of the attention backends on the pages
("sglang trtllm_mla_backend.py", TRTLLMMLABackend._run_decode_kernel and
forward_decode; "tokenspeed flashmla.py", FlashMLABackend.forward_decode):

* query        [B, q_len, H, 576]  -- absorbed latent part (512) then rope part (64)
* KV pool      [num_pages, page_size, 576], one latent head shared by all heads
* block table  int32 [B, W]; entries past a request's last page are unused
* seq_lens     int32 [B], counting the q_len new tokens

Draw order for one seed (numpy PCG64): sequence lengths, the page
permutation, the query, then the pool page by page.  Values are N(0, 1)
drawn in float32 and rounded to bf16 with round-to-nearest-even; the fp8
pool stores e4m3fn(clamp(x / k_scale, +-448)) (the per-tensor scale
convention of the pages' scaled_fp8_quant) and dequantises as code*k_scale.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

ROW_DIM = 576          # kv_lora_rank + qk_rope_head_dim
LATENT_DIM = 512       # kv_lora_rank = head_dim_v
ROPE_DIM = 64

# 1/sqrt(qk_nope_head_dim + qk_rope_head_dim) = 1/sqrt(128 + 64), as the fp32
# value a caller hands to the kernel.
SOFTMAX_SCALE_F32 = float(np.float32(1.0 / math.sqrt(192.0)))

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    heads: int
    page_size: int
    kv: str                      # "bf16" or "fp8"
    seed: int
    lens: tuple                  # ("fixed", [..]) | ("uniform", lo, hi) | ("lognormal", median, sigma, cap)
    num_pages: Optional[int] = None   # None: ceil(1.25 * pages in use)
    k_scale: float = 1.0
    min_work_units: int = 0      # 0: let the planner size the grid to the CU count
    ragged_q: bool = False       # per-request query lengths uniform in [1, q_len] (packed, see ragged())


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", batch=2, q_len=1, heads=16, page_size=64, kv="bf16", seed=1,
                 lens=("fixed", [100, 257]), num_pages=16),
        Workload("deepseek_decode", batch=64, q_len=1, heads=128, page_size=64, kv="bf16", seed=2,
                 lens=("uniform", 1024, 4096)),
        Workload("long_context", batch=8, q_len=1, heads=128, page_size=32, kv="bf16", seed=3,
                 lens=("lognormal", 8192, 1.0, 32768), min_work_units=512),
        Workload("mtp_verify", batch=128, q_len=4, heads=128, page_size=64, kv="bf16", seed=4,
                 lens=("uniform", 2048, 8192)),
        Workload("fp8_kv", batch=256, q_len=1, heads=128, page_size=64, kv="fp8", seed=5,
                 lens=("uniform", 512, 4096), k_scale=0.5),
        # the multi-token decode with a draft-extend batch's per-request query lengths
        Workload("draft_extend", batch=128, q_len=4, heads=128, page_size=64, kv="bf16", seed=6,
                 lens=("uniform", 2048, 8192), ragged_q=True),
    ]
}


@dataclasses.dataclass
class Inputs:
    """One decode call's inputs, as host arrays of raw storage bytes."""
    workload: Workload
    q: np.ndarray            # uint16 bf16 bits [B, q_len, H, 576]
    pool: np.ndarray         # uint16 bf16 bits or uint8 e4m3fn codes [N, P, 576]
    block_table: np.ndarray  # int32 [B, W]
    seq_lens: np.ndarray     # int32 [B]
    softmax_scale: float = SOFTMAX_SCALE_F32
    k_scale: float = 1.0

    @property
    def batch(self): return self.q.shape[0]
    @property
    def q_len(self): return self.q.shape[1]
    @property
    def heads(self): return self.q.shape[2]
    @property
    def page_size(self): return self.pool.shape[1]
    @property
    def num_pages(self): return self.pool.shape[0]
    @property
    def kv_fp8(self): return self.pool.dtype == np.uint8
    @property
    def max_seq_len(self): return int(self.seq_lens.max()) if self.seq_lens.size else 0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP float8_e4m3fn codes after clamping to +-448 (torch's CPU cast)."""
    import torch  # CPU cast only
    c = np.clip(np.asarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX)
    return torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def draw_seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.lens[0]
    if kind == "fixed":
        L = np.array(w.lens[1], dtype=np.int64)
    elif kind == "uniform":                       # integers, both ends inclusive
        L = rng.integers(w.lens[1], w.lens[2] + 1, size=w.batch)
    elif kind == "lognormal":                     # median * exp(sigma * z), capped; request 0 at the cap
        median, sigma, cap = w.lens[1], w.lens[2], w.lens[3]
        z = rng.standard_normal(w.batch)
        L = np.clip(np.rint(median * np.exp(sigma * z)), 1, cap).astype(np.int64)
        L[0] = cap
    else:
        raise ValueError(kind)
    assert L.shape == (w.batch,)
    return L.astype(np.int32)


def _fill_pool(rng, w: Workload, num_pages: int) -> np.ndarray:
    P = w.page_size
    if w.kv == "fp8":
        pool = np.empty((num_pages, P, ROW_DIM), dtype=np.uint8)
    else:
        pool = np.empty((num_pages, P, ROW_DIM), dtype=np.uint16)
    step = max(1, (1 << 24) // (P * ROW_DIM))    # about 16M values per draw
    for p0 in range(0, num_pages, step):
        p1 = min(num_pages, p0 + step)
        x = rng.standard_normal((p1 - p0, P, ROW_DIM), dtype=np.float32)
        if w.kv == "fp8":
            pool[p0:p1] = f32_to_e4m3fn_codes(x / np.float32(w.k_scale))
        else:
            pool[p0:p1] = f32_to_bf16_bits(x)
    return pool


def generate(w: Workload | str, seed: Optional[int] = None, poison: bool = False,
             seq_lens: Optional[np.ndarray] = None) -> Inputs:
    """Draw one call's inputs.  ``poison`` fills every pool slot no request
    reads (unused pages, tail slots of last pages) with NaN codes, to show the
    decode never reads them.  ``seq_lens`` overrides the drawn lengths (the
    draw still happens, so the rest of the stream is unchanged)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    L = draw_seq_lens(w, rng)
    if seq_lens is not None:
        L = np.asarray(seq_lens, dtype=np.int32).copy()
        assert L.shape == (w.batch,)
    P = w.page_size
    n = (L.astype(np.int64) + P - 1) // P
    used = int(n.sum())
    N = w.num_pages if w.num_pages is not None else int(math.ceil(1.25 * used))
    N = max(N, used, 1)
    perm = rng.permutation(N).astype(np.int32)
    W = max(1, int(n.max()) if n.size else 1)
    bt = np.full((w.batch, W), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        bt[b, :n[b]] = perm[off:off + n[b]]
        off += int(n[b])
    q = f32_to_bf16_bits(rng.standard_normal((w.batch, w.q_len, w.heads, ROW_DIM), dtype=np.float32))
    pool = _fill_pool(rng, w, N)
    inp = Inputs(w, q, pool, bt, L, SOFTMAX_SCALE_F32, float(w.k_scale) if w.kv == "fp8" else 1.0)
    if poison:
        poison_unused(inp)
    return inp


@dataclasses.dataclass
class Ragged:
    """A ragged multi-token batch: request b's q_b query tokens are rows
    qo_indptr[b] .. qo_indptr[b+1]-1 of the packed query (no padding)."""
    base: Inputs             # pool, block table, seq_lens; base.q is the padded [B, q_max, H, 576] draw
    q: np.ndarray            # uint16 bf16 bits [T, H, 576], T = qo_indptr[B]
    qo_indptr: np.ndarray    # int32 [B+1]
    q_lens: np.ndarray       # int32 [B]

    @property
    def total_q(self): return int(self.qo_indptr[-1])


def ragged(inp: Inputs, q_lens: Optional[np.ndarray] = None, seed: Optional[int] = None) -> Ragged:
    """Pack the first q_b query tokens of each request of ``inp`` (q_b drawn
    uniform in [1, q_len] from ``seed`` unless given; seq_lens are taken to
    count the q_b new tokens)."""
    B, qmax, H, D = inp.q.shape
    if q_lens is None:
        rng = np.random.default_rng(inp.workload.seed + 1000 if seed is None else seed)
        q_lens = rng.integers(1, qmax + 1, size=B)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    assert q_lens.shape == (B,) and (q_lens >= 0).all() and (q_lens <= qmax).all()
    indptr = np.zeros(B + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(q_lens)
    q = np.concatenate([inp.q[b, :q_lens[b]] for b in range(B)]) if B else np.zeros((0, H, D), np.uint16)
    return Ragged(inp, np.ascontiguousarray(q.reshape(-1, H, D)), indptr, q_lens)


def rope_cache(max_position: int, base: float = 10000.0, dim: int = ROPE_DIM) -> np.ndarray:
    """A rotary-embedding cos/sin cache [max_position, dim] float32: row p holds
    cos(p * f_i) in columns 0..dim/2-1 and sin(p * f_i) after them, with the
    frequencies f_i = base^(-2i/dim) of the original rotary embedding."""
    inv = base ** (-np.arange(0, dim, 2, dtype=np.float64) / dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def decode_positions(inp: Inputs) -> np.ndarray:
    """Positions [B, q_len] of each request's new query tokens: L_b - q_len + j
    (the cached tokens count the new ones)."""
    L = np.asarray(inp.seq_lens, dtype=np.int64)
    return np.maximum(L[:, None] - inp.q_len + np.arange(inp.q_len)[None, :], 0)


def poison_unused(inp: Inputs) -> None:
    """Write NaN into every pool slot that no request's visible tokens cover."""
    nan = FP8_NAN if inp.kv_fp8 else BF16_NAN
    P = inp.page_size
    live = np.zeros(inp.num_pages, dtype=bool)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        nb = (L + P - 1) // P
        live[inp.block_table[b, :nb]] = True
        if L % P:
            inp.pool[inp.block_table[b, nb - 1], L % P:, :] = nan
    inp.pool[~live] = nan


def permute_pages(inp: Inputs, seed: int) -> Inputs:
    """Same token rows, pool pages shuffled by a random permutation and the
    block table mapped through it."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(inp.num_pages).astype(np.int32)   # old page p -> new page sigma[p]
    pool = np.empty_like(inp.pool)
    pool[sigma] = inp.pool
    bt = np.where(inp.block_table >= 0, sigma[np.maximum(inp.block_table, 0)], inp.block_table).astype(np.int32)
    return dataclasses.replace(inp, pool=pool, block_table=bt)


def repack(inp: Inputs, page_size: int, seed: int) -> Inputs:
    """Same token rows of every request, stored with another page size in a
    freshly permuted pool."""
    rng = np.random.default_rng(seed)
    Pn = page_size
    L = inp.seq_lens.astype(np.int64)
    n = (L + Pn - 1) // Pn
    N = max(1, int(n.sum()))
    perm = rng.permutation(N).astype(np.int32)
    W = max(1, int(n.max()) if n.size else 1)
    bt = np.full((inp.batch, W), -1, dtype=np.int32)
    pool = np.zeros((N, Pn, ROW_DIM), dtype=inp.pool.dtype)
    off = 0
    for b in range(inp.batch):
        bt[b, :n[b]] = perm[off:off + n[b]]
        off += int(n[b])
        rows = gather_rows(inp, b)
        for t0 in range(0, int(L[b]), Pn):
            seg = rows[t0:t0 + Pn]
            pool[bt[b, t0 // Pn], :seg.shape[0]] = seg
    return dataclasses.replace(inp, pool=pool, block_table=bt)


def gather_rows(inp: Inputs, b: int) -> np.ndarray:
    """Raw stored rows [L_b, 576] of request b, in token order (byte copy)."""
    P = inp.page_size
    L = int(inp.seq_lens[b])
    t = np.arange(L)
    pages = inp.block_table[b, t // P]
    return inp.pool[pages, t % P]

"""Seeded random decode configurations on the GPU against the oracle: batch,
query length, head count, page size, ragged lengths (empty requests
included), pool type and k_scale, split mode -- drawn per seed, so that
combinations the hand-picked cases miss are covered too.  The same draws
drive ragged batches and the query read from two strided parts with the
rotary embedding, and the fp8 pool with the query cast to e4m3fn; a
medium-size family adds larger batches, head counts and lengths."""
import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
from oracle import ragged as RG, rope as R
import oracle_pins as P
from mla_synth import ragged, rope_cache
import gpu_util as G
from test_ragged import run_ragged
from test_q_fp8 import _oracle_q8, _run_q8


def _draw(seed):
    r = np.random.default_rng(7000 + seed)
    B = int(r.integers(1, 13))
    q_len = int(r.integers(1, 5))
    H = int(r.choice([1, 8, 16, 40, 64, 128]))
    Pg = int(r.choice([32, 64]))
    lens = r.integers(0, 700, size=B)
    lens[r.random(B) < 0.15] = 0
    kv = "fp8" if r.random() < 0.35 else "bf16"
    k_scale = float(r.choice([0.5, 0.25, 1.5])) if kv == "fp8" else None
    mode = r.choice(["auto", "forced", "units"])
    kw = {"auto": {}, "forced": {"num_splits": int(r.integers(1, 10))},
          "units": {"min_work_units": int(r.choice([r.integers(1, 64), r.integers(256, 3000)]))}}[mode]
    inp = P.small(kv=kv, q_len=q_len, heads=H, page_size=Pg, lens=tuple(int(x) for x in lens), seed=7000 + seed,
                  k_scale=k_scale)
    return inp, kw, r


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    inp, kw, _ = _draw(seed)
    o, l = G.run(inp, **kw)
    ro, rl = oracle.default().decode(inp)
    G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=f"seed {seed}: B={inp.batch} q={inp.q_len} H={inp.heads} "
                                                  f"P={inp.page_size} fp8={inp.kv_fp8} {kw}")


@pytest.mark.parametrize("seed", range(24))
def test_random_ragged(seed):
    inp, kw, r = _draw(100 + seed)
    q_lens = r.integers(0, inp.q_len + 1, size=inp.batch)
    rg = ragged(inp, q_lens=q_lens)
    o, l = run_ragged(rg, **kw)
    ro, rl = RG.decode(oracle.default(), rg)
    G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=f"ragged seed {seed}: q_lens={list(q_lens)} {kw}")


def _padded_view(t, head_major, pad_w, extra, dev="cuda"):
    """The values of t [T, H, W] as a strided view of a larger zero-filled
    buffer: each row padded by pad_w elements and `extra` unused token rows
    (or heads), tokens outermost or heads outermost."""
    T, H, W = t.shape
    if head_major:
        buf = torch.zeros((H, T + extra, W + pad_w), dtype=t.dtype, device=dev)
        v = buf[:, :T, :W].transpose(0, 1)
    else:
        buf = torch.zeros((T, H + extra, W + pad_w), dtype=t.dtype, device=dev)
        v = buf[:, :H, :W]
    v.copy_(t)
    return v


@pytest.mark.parametrize("seed", range(24))
def test_random_query_parts(seed):
    """The query as two strided parts (random padding, token- or head-major)
    with or without the rotary embedding (either pairing), at random
    positions, some outside the cos/sin cache (clamped): byte-identical to a
    plain decode of the oracle-rotated query, and within tolerance of the
    oracle's decode of it."""
    inp, kw, r = _draw(300 + seed)
    B, ql, H, _ = inp.q.shape
    T = B * ql
    rope = r.choice(["none", "neox", "interleaved"])
    q, pool, bt, sl = G.to_device(inp)
    qn = _padded_view(q[..., :512].reshape(T, H, 512), bool(r.random() < 0.5), 8 * int(r.integers(0, 4)),
                      int(r.integers(0, 3)))
    qr = _padded_view(q[..., 512:].reshape(T, H, 64), bool(r.random() < 0.5), 8 * int(r.integers(0, 9)),
                      int(r.integers(0, 3)))
    args = dict(max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale, k_scale=inp.k_scale, **kw)
    out1 = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse1 = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
    rq = inp.q
    if rope == "none":
        mla.mla_decode_qparts(qn, qr, pool, bt, sl, out1, lse1, **args)
    else:
        cache = rope_cache(int(inp.max_seq_len) + 8)
        pos = r.integers(-3, cache.shape[0] + 3, size=(B, ql)).astype(np.int64)
        mla.mla_decode_qparts(qn, qr, pool, bt, sl, out1, lse1,
                              positions=torch.from_numpy(pos.reshape(-1)).cuda(),
                              cos_sin_cache=torch.from_numpy(cache).cuda(), is_neox=rope == "neox", **args)
        rq = R.rotate_query(inp.q, np.clip(pos, 0, cache.shape[0] - 1), cache, rope == "neox")
    inp_r = dataclasses.replace(inp, q=rq)
    out2 = torch.full_like(out1, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    mla.mla_decode(torch.from_numpy(rq.view(np.int16)).view(torch.bfloat16).cuda(), pool, bt, sl, out2, lse2,
                   **args)
    torch.cuda.synchronize()
    what = f"seed {seed}: B={B} q={ql} H={H} fp8={inp.kv_fp8} rope={rope} strides={qn.stride()}/{qr.stride()} {kw}"
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32)), f"{what}: LSEs differ"
    ro, rl = oracle.default().decode(inp_r)
    G.compare(out1.float().cpu().numpy(), lse1.cpu().numpy(), ro, rl, fp8=inp.kv_fp8, what=what)


def _draw_fp8(seed):
    """The first of the draws 900 + 64*seed onwards that holds an fp8 pool
    (each does with probability 0.35, so one of 64 does but for ~1e-12)."""
    for s in range(900 + 64 * seed, 964 + 64 * seed):
        inp, kw, _ = _draw(s)
        if inp.kv_fp8:
            return inp, kw
    raise AssertionError(f"no fp8 draw among 64 from seed {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_query_fp8(seed):
    """The fp8 pool with the query cast to e4m3fn on random draws, against the
    oracle's decode of the cast query."""
    inp, kw = _draw_fp8(seed)
    o, l = _run_q8(inp, **kw)
    ro, rl = _oracle_q8(inp)
    G.compare(o, l, ro, rl, fp8=True, what=f"fp8 query seed {seed}: B={inp.batch} q={inp.q_len} H={inp.heads} {kw}")


def _draw_medium(seed):
    """Larger draws: up to 64 requests of 64 or 128 heads, up to 3000 tokens,
    so that split rows, the combine's grids and (ragged) row-block classes
    all occur."""
    r = np.random.default_rng(9100 + seed)
    B = int(r.integers(1, 65))
    q_len = int(r.integers(1, 5))
    H = int(r.choice([64, 128]))
    Pg = int(r.choice([32, 64]))
    lens = r.integers(0, 3000, size=B)
    lens[r.random(B) < 0.1] = 0
    kv = "fp8" if r.random() < 0.4 else "bf16"
    k_scale = float(r.choice([0.5, 1.5])) if kv == "fp8" else None
    mode = r.choice(["auto", "auto", "forced", "units"])
    kw = {"auto": {}, "forced": {"num_splits": int(r.integers(1, 12))},
          "units": {"min_work_units": int(r.choice([r.integers(1, 64), r.integers(256, 1500)]))}}[mode]
    inp = P.small(kv=kv, q_len=q_len, heads=H, page_size=Pg, lens=tuple(int(x) for x in lens), seed=9100 + seed,
                  k_scale=k_scale)
    return inp, kw, r


@pytest.mark.parametrize("seed", range(24))
def test_random_medium(seed):
    """Medium-size draws, in turn a uniform batch, a ragged one (random query
    lengths) and, for an fp8 pool, the query cast to e4m3fn."""
    inp, kw, r = _draw_medium(seed)
    kind = seed % 3
    what = f"medium seed {seed} kind {kind}: B={inp.batch} q={inp.q_len} H={inp.heads} P={inp.page_size} " \
           f"fp8={inp.kv_fp8} {kw}"
    if kind == 1:
        rg = ragged(inp, q_lens=r.integers(0, inp.q_len + 1, size=inp.batch))
        o, l = run_ragged(rg, **kw)
        ro, rl = RG.decode(oracle.default(), rg)
    elif kind == 2 and inp.kv_fp8:
        o, l = _run_q8(inp, **kw)
        ro, rl = _oracle_q8(inp)
    else:
        o, l = G.run(inp, **kw)
        ro, rl = oracle.default().decode(inp)
    G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=what)

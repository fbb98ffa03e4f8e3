"""The fp8 decode with the query cast to e4m3fn (quantize_q_fp8 = 1) vs the CPU
oracle, through the C ABI: the oracle decodes the query the pages' fp8 path
hands its kernel (oracle/query_fp8.py: each element's e4m3fn value, after the
rotation when one applies) against the same pool, in fp64.  The GPU's scores
are then exact products of e4m3fn values summed in fp32, so the fp8 tolerance
of the exact path holds unchanged."""
import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
from oracle import rope as R, ragged as RG
from oracle.query_fp8 import quantize_query
import oracle_pins as P
from mla_synth import generate, ragged, rope_cache, decode_positions
import gpu_util as G
from test_ragged import run_ragged


def _run_q8(inp, **kw):
    q, pool, bt, sl = G.to_device(inp)
    B, ql, H, _ = inp.q.shape
    out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
    args = dict(min_work_units=inp.workload.min_work_units)
    args.update(kw)
    mla.mla_decode(q, pool, bt, sl, out, lse, max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale,
                   k_scale=inp.k_scale, quantize_q_fp8=True, **args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_q8(inp):
    return oracle.default().decode(dataclasses.replace(inp, q=quantize_query(inp.q)))


CASES = [
    # q_len, heads, page, lens, k_scale
    (1, 128, 64, (1, 64, 65, 500), 0.5),
    (1, 16, 32, (0, 33, 100), 1.0),
    (4, 32, 64, (4, 70, 131), 0.25),
    (2, 40, 64, (2, 3, 97, 31), 1.5),
    (1, 256, 64, (1, 500), 0.5),
    (16, 256, 32, (16, 100, 300), 0.5),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", ["balanced", "balanced8", "split3"])
def test_small_cases(case, mode):
    ql, H, Pg, lens, ks = CASES[case]
    inp = P.small(kv="fp8", q_len=ql, heads=H, page_size=Pg, lens=lens, seed=500 + case, k_scale=ks)
    kw = dict(balanced=dict(), balanced8=dict(min_work_units=8), split3=dict(num_splits=3))[mode]
    o, l = _run_q8(inp, **kw)
    ro, rl = _oracle_q8(inp)
    G.compare(o, l, ro, rl, fp8=True, what=f"{CASES[case]} {mode}")


def test_query_holding_e4m3_values_is_unchanged():
    """A query whose elements are already e4m3fn values gives bit for bit the
    exact fp8 decode's scores up to the sum order, and the cast leaves it as it
    is: compare with the oracle on the same query."""
    inp = P.small(kv="fp8", q_len=2, heads=64, page_size=64, lens=(5, 90, 300), seed=520)
    inp = dataclasses.replace(inp, q=quantize_query(inp.q))
    o, l = _run_q8(inp)
    ro, rl = oracle.default().decode(inp)
    G.compare(o, l, ro, rl, fp8=True, what="pre-quantised query")


def test_differs_from_the_exact_path_by_the_cast():
    """The cast is what changes the scores: the exact fp8 path's output is
    farther from the quantised-query oracle than the fp8-product path's."""
    inp = P.small(kv="fp8", q_len=1, heads=128, page_size=64, lens=(400, 700), seed=521)
    o8, _ = _run_q8(inp)
    oe, _ = G.run(inp)
    ro, _ = _oracle_q8(inp)
    assert np.max(np.abs(o8 - ro)) < np.max(np.abs(oe - ro))


@pytest.mark.parametrize("is_neox", [True, False])
def test_with_rotation(is_neox):
    """qparts with the in-kernel rotation: the rope part is turned, rounded to
    bf16, then cast."""
    inp = P.small(kv="fp8", q_len=2, heads=32, page_size=64, lens=(0, 70, 131), seed=530, k_scale=0.5)
    B, ql, H, _ = inp.q.shape
    pos = decode_positions(inp)
    cache = rope_cache(int(inp.max_seq_len) + 8)
    q, pool, bt, sl = G.to_device(inp)
    T = B * ql
    qn, qr = q[..., :512].reshape(T, H, 512).contiguous(), q[..., 512:].reshape(T, H, 64).contiguous()
    out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_qparts(qn, qr, pool, bt, sl, out, lse, max_seq_len=inp.max_seq_len,
                          softmax_scale=inp.softmax_scale, k_scale=inp.k_scale,
                          positions=torch.from_numpy(np.ascontiguousarray(pos.reshape(-1), dtype=np.int64)).cuda(),
                          cos_sin_cache=torch.from_numpy(cache).cuda(), is_neox=is_neox, quantize_q_fp8=True)
    torch.cuda.synchronize()
    rq = quantize_query(R.rotate_query(inp.q, np.clip(pos, 0, cache.shape[0] - 1), cache, is_neox))
    ro, rl = oracle.default().decode(dataclasses.replace(inp, q=rq))
    G.compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, fp8=True, what=f"rotation neox={is_neox}")


@pytest.mark.parametrize("mode", ["balanced", "split3"])
def test_ragged(mode):
    inp = P.small(kv="fp8", q_len=4, heads=32, page_size=64, lens=(4, 70, 131, 0, 260), seed=540, k_scale=0.5)
    rg = ragged(inp, q_lens=(2, 4, 1, 0, 3))
    kw = dict(balanced=dict(), split3=dict(num_splits=3))[mode]
    o, l = run_ragged(rg, quantize_q_fp8=True, **kw)
    ro, rl = RG.decode(oracle.default(), dataclasses.replace(rg, q=quantize_query(rg.q)))
    T = rg.q.shape[0]
    G.compare(o[:T], l[:T], ro, rl, fp8=True, what=f"ragged {mode}")


def test_full_size_fp8_workload_whole():
    """The fp8 workload (256 requests of 512..4096 tokens, 128 heads) with the
    cast, every query row against the oracle."""
    inp = generate("fp8_kv")
    o, l = _run_q8(inp)
    ro, rl = _oracle_q8(inp)
    rel = G.compare(o, l, ro, rl, fp8=True, what="fp8_kv with the query cast")
    print(f"fp8_kv quantised query: max|gpu-oracle|/max|oracle| = {rel:.3e}, max|lse err| = {G.lse_err(l, rl):.3e}")


def test_bf16_pool_rejects_the_cast():
    inp = P.small(kv="bf16", q_len=1, heads=16, page_size=64, lens=(5,), seed=550)
    q, pool, bt, sl = G.to_device(inp)
    out = torch.empty((1, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError):
        mla.mla_decode(q, pool, bt, sl, out, None, max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale,
                       quantize_q_fp8=True)

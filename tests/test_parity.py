"""GPU decode vs the CPU oracle (through the C ABI), element by element.

Small inputs and the full-size workloads (in the launch configuration the
benchmark times) are compared over their whole output; a sampled check of the
full-size workloads runs first as a quick pre-check, and properties that hold
at any size (repeatability) follow."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle
from oracle import ragged as RG
import oracle_pins as P
from mla_synth import generate, WORKLOADS, ragged
import gpu_util as G
from test_ragged import run_ragged


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def test_tiny_workload(orc):
    inp = generate("tiny")
    o, l = G.run(inp)
    ro, rl = orc.decode(inp)
    G.compare(o, l, ro, rl, what="tiny")


CASES = [
    # kv, q_len, heads, page, lens
    ("bf16", 1, 16, 64, (1, 31, 32, 33, 63, 64, 65, 100, 257)),
    ("bf16", 1, 128, 32, (5, 300, 1000)),
    ("bf16", 1, 64, 64, (0, 1, 2, 129)),
    ("bf16", 1, 1, 32, (40, 90)),
    ("bf16", 1, 48, 64, (77, 1)),
    ("bf16", 4, 128, 64, (4, 5, 67, 300)),
    ("bf16", 2, 16, 32, (1, 2, 3, 40)),
    ("bf16", 3, 40, 64, (2, 3, 97)),
    ("fp8", 1, 128, 64, (1, 64, 65, 500)),
    ("fp8", 1, 16, 32, (0, 33, 100)),
    ("fp8", 4, 32, 64, (4, 70, 131)),
    # the limits the library accepts: q_len * heads = 4096 query rows (64 row
    # blocks per request), the longest q_len, the most heads
    ("bf16", 16, 256, 64, (16, 100, 300)),
    ("bf16", 64, 64, 32, (64, 65, 200)),
    ("fp8", 1, 256, 64, (1, 500)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", ["balanced", "balanced8", "split3"])
def test_small_cases(orc, case, mode):
    kv, ql, H, Pg, lens = CASES[case]
    inp = P.small(kv=kv, q_len=ql, heads=H, page_size=Pg, lens=lens, seed=100 + case)
    kw = dict(balanced=dict(), balanced8=dict(min_work_units=8), split3=dict(num_splits=3))[mode]
    o, l = G.run(inp, **kw)
    ro, rl = orc.decode(inp)
    G.compare(o, l, ro, rl, fp8=kv == "fp8", what=f"{CASES[case]} {mode}")


def _sample_rows(inp, n_per_req, seed):
    rng = np.random.default_rng(seed)
    sel = []
    for b in range(inp.batch):
        for _ in range(n_per_req):
            sel.append((b, int(rng.integers(inp.q_len)), int(rng.integers(inp.heads))))
        sel.append((b, inp.q_len - 1, inp.heads - 1))
    return sel


@pytest.mark.parametrize("name", ["deepseek_decode", "long_context", "mtp_verify", "fp8_kv"])
def test_full_size_workload_sampled(orc, name):
    inp = generate(name)
    o, l = G.run(inp)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    per = {"deepseek_decode": 4, "long_context": 24, "mtp_verify": 1, "fp8_kv": 1}[name]
    sel = _sample_rows(inp, per, seed=7)
    ro, rl = orc.decode_rows(inp, sel)
    go = np.stack([o[b, j, h] for b, j, h in sel])
    gl = np.array([l[b, j, h] for b, j, h in sel])
    G.compare(go, gl, ro, rl, fp8=inp.kv_fp8, what=name)


@pytest.mark.parametrize("name", ["deepseek_decode", "long_context", "mtp_verify", "fp8_kv"])
def test_full_size_workload_whole(orc, name):
    """Every query row of the full-size workload, in the launch configuration
    the benchmark times (the workload's own planner target), against the fp64
    oracle over the whole output: one global max|gpu - oracle| against the
    largest |oracle| value of the tensor, and every LSE."""
    inp = generate(name)
    o, l = G.run(inp)
    ro, rl = orc.decode(inp)
    rel = G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=name)
    lerr = G.lse_err(l, rl)
    print(f"{name}: {o.shape[0] * o.shape[1] * o.shape[2]} rows, max|gpu-oracle|/max|oracle| = {rel:.3e}, "
          f"max|lse err| = {lerr:.3e}")


@pytest.mark.parametrize("name", ["deepseek_decode", "long_context", "fp8_kv"])
def test_full_size_repeatable(name):
    """Many back-to-back calls on the same inputs give bit-identical outputs and
    LSEs.  This guards the LDS hand-offs between the waves of a workgroup (the
    softmax weights, the row statistics, the staged output rows): a write that
    is still in flight at a barrier shows up as an occasional wrong row group."""
    import paged_mla_decode_06_amd as mla
    inp = generate(name)
    q, pool, bt, sl = G.to_device(inp)
    B, ql, H, _ = inp.q.shape
    p = mla.params_for(q, pool, bt, inp.max_seq_len, inp.softmax_scale, inp.k_scale,
                       min_work_units=inp.workload.min_work_units)
    ws = mla.alloc_workspace(p, q.device)
    ref_o = torch.empty((B, ql, H, 512), dtype=torch.bfloat16, device=q.device)
    ref_l = torch.empty((B, ql, H), dtype=torch.float32, device=q.device)
    mla.mla_decode_timed(p, q, pool, bt, sl, ref_o, ref_l, ws, None, None, None, None)
    outs = [torch.empty_like(ref_o) for _ in range(8)]
    lses = [torch.empty_like(ref_l) for _ in range(8)]
    differing = []
    for it in range(160):
        o, l = outs[it % 8], lses[it % 8]
        mla.mla_decode_timed(p, q, pool, bt, sl, o, l, ws, None, None, None, None)
        if it % 8 == 7:
            torch.cuda.synchronize()
            for k in range(8):
                same = bool(torch.equal(outs[k].view(torch.int16), ref_o.view(torch.int16))) and \
                    bool(torch.equal(lses[k].view(torch.int32), ref_l.view(torch.int32)))
                if not same:
                    rows = (outs[k].view(torch.int16) != ref_o.view(torch.int16)).any(dim=-1).nonzero()
                    differing.append((it - 7 + k, rows[:4].tolist()))
    assert not differing, f"{name}: {len(differing)} of 160 calls differ from the first, e.g. {differing[:3]}"


@pytest.mark.parametrize("B", [700, 1024, 1025, 1500, 8192])
def test_many_requests(orc, B):
    """Large batches of short requests, some empty: the workgroup plan is found
    by one wave per workgroup up to 1024 requests and block-wide beyond (both
    sides of that boundary are taken), up to 8192, the largest batch the
    library accepts (its offsets then fill 32 KB of the tile buffers)."""
    rng = np.random.default_rng(50 + B)
    lens = rng.integers(0, 70, size=B)
    lens[::97] = 0
    inp = P.small(lens=tuple(int(x) for x in lens), heads=16, seed=51)
    ro, rl = orc.decode(inp)
    o, l = G.run(inp)
    G.compare(o, l, ro, rl, what=f"B={B}")


def test_many_requests_fp8_multi_token(orc):
    """1024 requests (the most the combine's group grid takes), fp8 cache,
    two query tokens each, some empty: fewer groups than requests."""
    rng = np.random.default_rng(52)
    lens = rng.integers(0, 300, size=1024)
    lens[::61] = 0
    inp = P.small(kv="fp8", q_len=2, lens=tuple(int(x) for x in lens), heads=16, seed=53, k_scale=0.5)
    o, l = G.run(inp)
    ro, rl = orc.decode(inp)
    G.compare(o, l, ro, rl, fp8=True, what="B=1024 fp8 q_len=2")


def test_many_requests_ragged(orc):
    """1000 ragged requests with 0 to 4 query tokens through the group grid."""
    rng = np.random.default_rng(54)
    lens = rng.integers(4, 400, size=1000)
    inp = P.small(q_len=4, lens=tuple(int(x) for x in lens), heads=16, seed=55)
    rg = ragged(inp, q_lens=rng.integers(0, 5, size=1000))
    o, l = run_ragged(rg)
    ro, rl = RG.decode(orc, rg)
    G.compare(o, l, ro, rl, what="B=1000 ragged")

"""The decode step under HIP graph capture: the launch shape depends only on
host-side parameters (batch, heads, q_len, page size, the max_seq_len bound,
the CU count), and the split plan is rebuilt inside the kernel from the
device seq_lens, so one captured graph serves every step whose lengths stay
within the bound.  Each replay, with new lengths, block tables and rows and
with eager work between replays, must give the bytes an eager call gives."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
from mla_synth import Workload, generate


def _inputs(seed, lens, max_len):
    w = Workload(name="graph", batch=len(lens), q_len=2, heads=128, page_size=64, kv="bf16", seed=seed,
                 lens=("fixed", list(lens)), num_pages=(max_len // 64 + 1) * len(lens) + 4)
    inp = generate(w)
    bt = np.full((len(lens), max_len // 64 + 1), -1, dtype=np.int32)
    bt[:, :inp.block_table.shape[1]] = inp.block_table
    return inp, bt


def test_decode_step_graph_replays_match_eager():
    B, max_len = 12, 3000
    rng = np.random.default_rng(70)
    inp, bt = _inputs(71, rng.integers(2, max_len + 1, size=B), max_len)
    dev = "cuda"
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    pool = torch.from_numpy(inp.pool.view(np.int16)).view(torch.bfloat16).to(dev)
    bt_d = torch.from_numpy(bt).to(dev)
    sl_d = torch.from_numpy(inp.seq_lens).to(dev)
    out = torch.zeros((B, 2, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B, 2, 128), dtype=torch.float32, device=dev)
    # the appended rows of the step: the newest token of each request
    new_rows = torch.empty((B, 576), dtype=torch.bfloat16, device=dev)
    new_locs = torch.empty(B, dtype=torch.int64, device=dev)
    p = mla.make_params(B, 2, 128, 64, inp.num_pages, bt.shape[1], max_len, softmax_scale=inp.softmax_scale)
    ws = mla.alloc_workspace(p, dev)

    def step(stream=None):
        mla.mla_kv_append(new_rows[:, :512], new_rows[:, 512:], new_locs, pool, stream=stream)
        mla.mla_decode(q, pool, bt_d, sl_d, out, lse, ws, max_seq_len=max_len, softmax_scale=inp.softmax_scale,
                       stream=stream, params=p)

    def set_step(seed):
        r = np.random.default_rng(seed)
        lens = r.integers(2, max_len + 1, size=B).astype(np.int32)
        inp2, bt2 = _inputs(seed, lens, max_len)
        q.copy_(torch.from_numpy(inp2.q.view(np.int16)).view(torch.bfloat16))
        pool.copy_(torch.from_numpy(inp2.pool.view(np.int16)).view(torch.bfloat16))
        bt_d.copy_(torch.from_numpy(bt2))
        sl_d.copy_(torch.from_numpy(lens))
        new_rows.normal_()
        locs = [int(bt2[b, (L - 1) // 64]) * 64 + (L - 1) % 64 for b, L in enumerate(lens)]
        new_locs.copy_(torch.tensor(locs, dtype=torch.int64))
        return pool.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()          # eager warm-up on the capture stream (first-use attributes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for k in range(4):
        pool0 = set_step(100 + k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        go, gl, gp = out.clone(), lse.clone(), pool.clone()
        pool.copy_(pool0)
        out.zero_()
        lse.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(gp.view(torch.int16), pool.view(torch.int16)), f"replay {k}: pool differs"
        assert torch.equal(go.view(torch.int16), out.view(torch.int16)), f"replay {k}: output differs"
        assert torch.equal(gl.view(torch.int32), lse.view(torch.int32)), f"replay {k}: lse differs"

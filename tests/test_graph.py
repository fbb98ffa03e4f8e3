"""The decode step under HIP graph capture: the launch shape depends only on
host-side parameters (batch, heads, q_len, page size, the max_seq_len bound,
the CU count), and the split plan is rebuilt inside the kernel from the
device seq_lens, so one captured graph serves every step whose lengths stay
within the bound.

The step is the KV append followed by the decode.  Each replay, with new
lengths, block tables, query and appended rows, and with eager work between
replays, must give the bytes an eager call gives, and the output of the
oracle (the oracle's append, then the oracle's decode) on that step's inputs.

Batches smaller than the captured one are padded as the pages pad them: the
graph is captured per batch size, the block-table buffer starts zeroed, and a
padding row's sequence length is the capture fill value 1
("tokenspeed trtllm_mla.py", TRTLLMMLABackend.init_cuda_graph_state,
init_forward_metadata_capture_cuda_graph / init_forward_metadata_replay_cuda_graph
and get_cuda_graph_seq_len_fill_value; "sglang trtllm_mla_backend.py",
_apply_cuda_graph_metadata).  Page 0 is the padding page no live request
owns, and a padding row appends nothing (its location is -1).  A padding row
with length 0 is covered too."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
from oracle import kv_append as KA
from mla_synth import Workload, generate
from mla_synth.gen import f32_to_bf16_bits
import gpu_util as G

B_CAP, Q_LEN, HEADS, PAGE, MAX_LEN = 12, 2, 128, 64, 3000
W = MAX_LEN // PAGE + 1


def _step(seed, live, pad_len=1):
    """Host inputs of one decode step at the captured batch size: `live`
    requests drawn by the generator (pages shifted up by one, so page 0 is
    the padding page), then B_CAP - live padding rows of length pad_len with
    an all-zero block-table row.  Returns a generator-like input object for
    the oracle plus the appended rows and their locations."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(2, MAX_LEN + 1, size=live)
    w = Workload(name="graph", batch=live, q_len=Q_LEN, heads=HEADS, page_size=PAGE, kv="bf16", seed=seed,
                 lens=("fixed", [int(x) for x in lens]), num_pages=W * B_CAP + 4)
    inp = generate(w)
    N = inp.num_pages + 1
    pool = np.empty((N, PAGE, 576), dtype=np.uint16)
    pool[1:] = inp.pool
    pool[0] = f32_to_bf16_bits(rng.standard_normal((PAGE, 576)).astype(np.float32))
    bt = np.zeros((B_CAP, W), dtype=np.int32)
    used = inp.block_table >= 0
    bt[:live, :inp.block_table.shape[1]] = np.where(used, inp.block_table + 1, -1)
    sl = np.full(B_CAP, pad_len, dtype=np.int32)
    sl[:live] = inp.seq_lens
    q = np.empty((B_CAP, Q_LEN, HEADS, 576), dtype=np.uint16)
    q[:live] = inp.q
    q[live:] = f32_to_bf16_bits(rng.standard_normal((B_CAP - live, Q_LEN, HEADS, 576)).astype(np.float32))
    rows = f32_to_bf16_bits(rng.standard_normal((B_CAP, 576)).astype(np.float32))
    locs = np.full(B_CAP, -1, dtype=np.int64)
    for b in range(live):
        L = int(sl[b])
        locs[b] = int(bt[b, (L - 1) // PAGE]) * PAGE + (L - 1) % PAGE
    full = type(inp)(workload=inp.workload, q=q, pool=pool, block_table=bt, seq_lens=sl,
                     softmax_scale=inp.softmax_scale, k_scale=inp.k_scale)
    return full, rows, locs


def test_decode_step_graph_replays_match_eager_and_oracle():
    dev = "cuda"
    first, _, _ = _step(100, B_CAP)
    N = first.num_pages
    q = torch.empty((B_CAP, Q_LEN, HEADS, 576), dtype=torch.bfloat16, device=dev)
    pool = torch.empty((N, PAGE, 576), dtype=torch.bfloat16, device=dev)
    bt_d = torch.zeros((B_CAP, W), dtype=torch.int32, device=dev)
    sl_d = torch.ones(B_CAP, dtype=torch.int32, device=dev)
    out = torch.zeros((B_CAP, Q_LEN, HEADS, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B_CAP, Q_LEN, HEADS), dtype=torch.float32, device=dev)
    new_rows = torch.empty((B_CAP, 576), dtype=torch.bfloat16, device=dev)
    new_locs = torch.full((B_CAP,), -1, dtype=torch.int64, device=dev)
    p = mla.make_params(B_CAP, Q_LEN, HEADS, PAGE, N, W, MAX_LEN, softmax_scale=first.softmax_scale)
    ws = mla.alloc_workspace(p, dev)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)

    def load(inp, rows, locs):
        q.copy_(to_dev(inp.q))
        pool.copy_(to_dev(inp.pool))
        bt_d.copy_(torch.from_numpy(inp.block_table))
        sl_d.copy_(torch.from_numpy(inp.seq_lens))
        new_rows.copy_(to_dev(rows))
        new_locs.copy_(torch.from_numpy(locs))

    def step(stream=None):
        mla.mla_kv_append(new_rows[:, :512], new_rows[:, 512:], new_locs, pool, stream=stream)
        mla.mla_decode(q, pool, bt_d, sl_d, out, lse, ws, max_seq_len=MAX_LEN, softmax_scale=first.softmax_scale,
                       stream=stream, params=p)

    load(*_step(99, B_CAP))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()          # eager warm-up on the capture stream (first-use attributes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())

    orc = oracle.default()
    # (seed, live requests, padding length): full batches, then smaller live
    # batches padded to the captured size
    for k, (seed, live, pad_len) in enumerate([(100, B_CAP, 1), (101, B_CAP, 1), (102, 7, 1), (103, 5, 0),
                                               (104, 1, 1)]):
        inp, rows, locs = _step(seed, live, pad_len)
        load(inp, rows, locs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        go, gl, gp = out.clone(), lse.clone(), pool.clone()
        # the oracle: its own append of the step's rows, then its decode
        ref_pool = KA.kv_append(inp.pool, rows[:, :512], rows[:, 512:], locs)
        assert np.array_equal(gp.view(torch.int16).cpu().numpy().view(np.uint16), ref_pool), \
            f"replay {k}: pool differs from the oracle's append"
        ref_inp = type(inp)(workload=inp.workload, q=inp.q, pool=ref_pool, block_table=inp.block_table,
                            seq_lens=inp.seq_lens, softmax_scale=inp.softmax_scale, k_scale=inp.k_scale)
        ro, rl = orc.decode(ref_inp)
        G.compare(go.float().cpu().numpy(), gl.cpu().numpy(), ro, rl,
                  what=f"replay {k} (live {live}, padding length {pad_len})")
        # eager call on the same inputs: the same bytes
        load(inp, rows, locs)
        out.zero_()
        lse.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(gp.view(torch.int16), pool.view(torch.int16)), f"replay {k}: pool differs from eager"
        assert torch.equal(go.view(torch.int16), out.view(torch.int16)), f"replay {k}: output differs from eager"
        assert torch.equal(gl.view(torch.int32), lse.view(torch.int32)), f"replay {k}: lse differs from eager"

"""GPU ragged multi-token decode (mla_decode_ragged) vs the CPU oracle, through
the C ABI: per-request query lengths packed by offsets, including requests
with no query token; bit-identical to mla_decode when every length is the
same; offsets outside the query tensor are ignored, not followed."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
from oracle import ragged as RG
import oracle_pins as P
from mla_synth import generate, ragged
import gpu_util as G


def run_ragged(rg, total_q=None, guard=0, **kw):
    inp = rg.base
    _, pool, bt, sl = G.to_device(inp)
    T, H, _ = rg.q.shape
    q = torch.from_numpy(rg.q.view(np.int16)).view(torch.bfloat16).cuda()
    ind = torch.from_numpy(rg.qo_indptr).cuda()
    out_full = torch.full((T + guard, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_full = torch.full((T + guard, H), float("nan"), dtype=torch.float32, device="cuda")
    Tq = T if total_q is None else total_q
    q_use = q if total_q is None else q[:total_q]
    args = dict(max_q_len=inp.q_len, max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale,
                k_scale=inp.k_scale, min_work_units=inp.workload.min_work_units)
    args.update(kw)
    mla.mla_decode_ragged(q_use.contiguous(), ind, pool, bt, sl, out_full[:Tq], lse_full[:Tq], **args)
    torch.cuda.synchronize()
    return out_full.float().cpu().numpy(), lse_full.cpu().numpy()


CASES = [
    # kv, q_max, heads, page, lens, q_lens
    ("bf16", 4, 128, 64, (4, 5, 67, 300, 130), (1, 4, 2, 3, 4)),
    ("bf16", 4, 16, 32, (1, 2, 3, 40, 64, 65), (1, 2, 0, 4, 3, 1)),
    ("bf16", 3, 40, 64, (2, 3, 97), (3, 1, 2)),
    ("bf16", 8, 16, 32, (8, 100, 33), (8, 5, 1)),
    ("fp8", 4, 32, 64, (4, 70, 131, 0), (2, 4, 1, 0)),
    ("fp8", 2, 128, 32, (5, 300), (2, 1)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", ["balanced", "balanced8", "split3"])
def test_small_cases(case, mode):
    kv, qmax, H, Pg, lens, qls = CASES[case]
    inp = P.small(kv=kv, q_len=qmax, heads=H, page_size=Pg, lens=lens, seed=200 + case)
    rg = ragged(inp, q_lens=qls)
    kw = dict(balanced=dict(), balanced8=dict(min_work_units=8), split3=dict(num_splits=3))[mode]
    o, l = run_ragged(rg, **kw)
    ro, rl = RG.decode(oracle.default(), rg)
    G.compare(o, l, ro, rl, fp8=kv == "fp8", what=f"{CASES[case]} {mode}")


def test_uniform_lengths_identical_to_mla_decode():
    inp = P.small(kv="bf16", q_len=4, heads=128, page_size=64, lens=(4, 67, 300, 1000), seed=210)
    rg = ragged(inp, q_lens=[4, 4, 4, 4])
    o, l = run_ragged(rg)
    uo, ul = G.run(inp)
    assert np.array_equal(o.reshape(uo.shape).view(np.uint32), uo.view(np.uint32))
    assert np.array_equal(l.reshape(ul.shape).view(np.uint32), ul.view(np.uint32))


def test_offsets_past_the_query_are_ignored():
    """total_q below the last offset: the last request is treated as having no
    query token; nothing is written past row total_q (guard rows stay NaN)."""
    inp = P.small(kv="bf16", q_len=3, heads=16, page_size=32, lens=(10, 40, 70), seed=211)
    rg = ragged(inp, q_lens=[2, 3, 3])
    o, l = run_ragged(rg, total_q=5, guard=3)
    ro, rl = RG.decode(oracle.default(), rg)
    G.compare(o[:5], l[:5], ro[:5], rl[:5], what="first two requests")
    assert np.isnan(o[5:]).all() and np.isnan(l[5:]).all()


def test_no_query_token_in_the_batch():
    """Every request with q_b = 0: an empty query and output, a no-op call."""
    inp = P.small(kv="fp8", q_len=2, heads=64, page_size=32, lens=(686, 159), seed=212, k_scale=0.5)
    rg = ragged(inp, q_lens=[0, 0])
    o, l = run_ragged(rg)
    assert o.shape == (0, 64, 512) and l.shape == (0, 64)


def test_full_size_draft_extend_sampled():
    """The MTP-shaped batch with per-request lengths uniform in [1, 4], in the
    launch configuration the benchmark times, on sampled rows."""
    rg = ragged(generate("draft_extend"))
    o, l = run_ragged(rg)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    rng = np.random.default_rng(9)
    sel = [(int(rng.integers(rg.total_q)), int(rng.integers(128))) for _ in range(96)]
    sel += [(int(rg.qo_indptr[b + 1]) - 1, 127) for b in range(0, rg.base.batch, 9)]
    ro, rl = RG.decode_rows(oracle.default(), rg, sel)
    G.compare(np.stack([o[t, h] for t, h in sel]), np.array([l[t, h] for t, h in sel]), ro, rl,
              what="draft_extend")


def test_full_size_draft_extend_whole():
    """The whole draft-extend batch (every packed query row and head) against
    the fp64 oracle, in the launch configuration the benchmark times."""
    rg = ragged(generate("draft_extend"))
    o, l = run_ragged(rg)
    ro, rl = RG.decode(oracle.default(), rg)
    rel = G.compare(o, l, ro, rl, what="draft_extend")
    print(f"draft_extend: {o.shape[0] * o.shape[1]} rows, max|gpu-oracle|/max|oracle| = {rel:.3e}, "
          f"max|lse err| = {G.lse_err(l, rl):.3e}")


def test_offsets_beyond_max_q_len_leave_rows_untouched():
    """A request with more query tokens than max_q_len: its first max_q_len
    tokens are decoded (as if it had that many), the rows of the rest are not
    written; validate=True rejects the offsets before any device work."""
    inp = P.small(kv="bf16", q_len=5, heads=16, page_size=32, lens=(40, 90), seed=212)
    rg = ragged(inp, q_lens=[5, 2])          # request 0 has 5 tokens, max_q_len below is 4
    _, pool, bt, sl = G.to_device(inp)
    T, H, _ = rg.q.shape
    q = torch.from_numpy(rg.q.view(np.int16)).view(torch.bfloat16).cuda()
    ind = torch.from_numpy(rg.qo_indptr).cuda()
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    args = dict(max_q_len=4, max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_ragged(q, ind, pool, bt, sl, out, lse, validate=True, **args)
    assert e.value.status == mla.MLA_ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a rejected call writes nothing"
    mla.mla_decode_ragged(q, ind, pool, bt, sl, out, lse, **args)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isnan(o[4]).all() and np.isnan(l[4]).all(), "the token past max_q_len must stay unwritten"
    # the first four tokens of request 0 are decoded as a 4-token request of
    # the same length: token j sees t < L - 4 + 1 + j
    v = RG.request_view(rg, 0)
    v.q = np.ascontiguousarray(v.q[:, :4])
    v.q_len = 4
    ro, rl = oracle.default().decode(v)
    G.compare(o[:4], l[:4], ro[0], rl[0], what="request 0, first four tokens")
    ro1, rl1 = RG.decode(oracle.default(), rg)
    G.compare(o[5:], l[5:], ro1[5:], rl1[5:], what="request 1")


# Ragged batches that the row-block class plan takes (balanced mode, at most 8
# row blocks, requests with fewer than all of them): the plan is confirmed on
# the host mirror, then the decode is compared with the oracle over the whole
# output.  (kv, q_max, heads, page, batch, max length, query lengths: None =
# random in 0..q_max, or one value for every request, seed)
CLASS_CASES = [
    ("bf16", 4, 128, 64, 40, 1500, None, 301),
    ("fp8", 2, 128, 32, 33, 900, None, 302),
    ("bf16", 4, 128, 64, 24, 2000, 1, 303),      # one class below nrb only
    ("bf16", 8, 64, 64, 30, 1200, None, 304),     # eight row blocks of 64 heads x 8 tokens
    ("bf16", 2, 128, 64, 1100, 200, None, 305),   # more requests than the workgroup has threads
]


@pytest.mark.parametrize("case", range(len(CLASS_CASES)))
def test_class_plan_cases(case):
    kv, qmax, H, Pg, B, maxlen, ql, seed = CLASS_CASES[case]
    rng = np.random.default_rng(seed)
    lens = tuple(int(x) for x in rng.integers(0, maxlen + 1, size=B))
    inp = P.small(kv=kv, q_len=qmax, heads=H, page_size=Pg, lens=lens, seed=seed,
                  k_scale=0.5 if kv == "fp8" else None)
    q_lens = rng.integers(0, qmax + 1, size=B) if ql is None else np.full(B, ql)
    rg = ragged(inp, q_lens=q_lens)
    p = mla.make_params(B, qmax, H, Pg, inp.num_pages, inp.block_table.shape[1], inp.max_seq_len,
                        mla.MLA_KV_FP8_E4M3FN if inp.kv_fp8 else mla.MLA_KV_BF16, inp.softmax_scale,
                        inp.k_scale, 0, 0, 0)
    _, _, used = mla.mla_plan_host_ragged(p, inp.seq_lens, rg.qo_indptr, int(rg.qo_indptr[-1]))
    assert used, "the class plan should apply to this batch"
    o, l = run_ragged(rg)
    ro, rl = RG.decode(oracle.default(), rg)
    G.compare(o, l, ro, rl, fp8=kv == "fp8", what=f"class plan case {case}")

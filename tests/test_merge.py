"""Split row blocks merged by the combine kernel, against the oracle for
2 to 8 pieces per row block; and a workspace shared by calls of different
parameters: each call's result is bit-identical to the same call on a fresh
workspace (a call reads only workspace bytes it has written)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
import oracle_pins as P
from mla_synth import generate
import gpu_util as G


def _call(inp, ws, **kw):
    q, pool, bt, sl = G.to_device(inp)
    B, ql, H, _ = inp.q.shape
    out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
    args = dict(max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale, k_scale=inp.k_scale,
                min_work_units=inp.workload.min_work_units)
    args.update(kw)
    mla.mla_decode(q, pool, bt, sl, out, lse, ws, **args)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_forced_pieces_against_oracle(splits, kv):
    """Requests shorter than the split count have fewer pieces."""
    inp = P.small(kv=kv, q_len=2, heads=64, page_size=64, lens=(1, 40, 97, 300, 129), seed=600 + splits)
    o, l = G.run(inp, num_splits=splits)
    ro, rl = oracle.default().decode(inp)
    G.compare(o, l, ro, rl, fp8=kv == "fp8", what=f"{kv} num_splits={splits}")


def test_workspace_shared_by_calls_of_different_parameters():
    big = generate("deepseek_decode")
    cases = [(big, {}),
             (P.small(kv="fp8", q_len=2, heads=32, page_size=32, lens=(1, 40, 300, 0, 77), seed=610), dict(num_splits=3)),
             (P.small(kv="bf16", q_len=1, heads=128, page_size=64, lens=(900, 33, 2000), seed=611), dict(min_work_units=8)),
             (big, {})]
    need = max(mla.mla_decode_workspace_size(mla.params_for(*G.to_device(inp)[:3], inp.max_seq_len,
                                                            inp.softmax_scale, inp.k_scale, **kw))
               for inp, kw in cases)
    shared = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for i, (inp, kw) in enumerate(cases):
        o1, l1 = _call(inp, shared, **kw)
        fresh = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
        o2, l2 = _call(inp, fresh, **kw)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"call {i}: output depends on the workspace's past"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"call {i}: lse depends on the workspace's past"

"""GPU decode with the query given as its two parts (mla_decode_qparts):
the latent part and the rope part read in place through their own token
and head strides, bit-identical to mla_decode on the concatenated query,
and within the bar of the oracle."""
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


def _parts(q, layout):
    """q [B, q_len, H, 576] on the GPU -> (q_nope, q_rope) in the given layout."""
    B, ql, H, _ = q.shape
    T = B * ql
    if layout == "slices":                 # two views of one tensor
        return q[..., :512], q[..., 512:]
    if layout == "separate":               # two contiguous tensors [T, H, w]
        return q[..., :512].reshape(T, H, 512).contiguous(), q[..., 512:].reshape(T, H, 64).contiguous()
    if layout == "head_major":             # the absorbed product's [H, T, 512] output seen token-major
        nope = q[..., :512].reshape(T, H, 512).transpose(0, 1).contiguous().transpose(0, 1)
        rope_buf = torch.zeros((T, H, 128), dtype=q.dtype, device=q.device)   # padded head stride 128
        rope_buf[..., :64] = q[..., 512:].reshape(T, H, 64)
        return nope, rope_buf[..., :64]
    raise ValueError(layout)


def _both(inp, layout, **kw):
    q, pool, bt, sl = G.to_device(inp)
    B, ql, H, _ = inp.q.shape
    outs = []
    for use_parts in (False, True):
        out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
        args = dict(max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale, k_scale=inp.k_scale,
                    min_work_units=inp.workload.min_work_units, **kw)
        if use_parts:
            qn, qr = _parts(q, layout)
            mla.mla_decode_qparts(qn, qr, pool, bt, sl, out, lse, **args)
        else:
            mla.mla_decode(q, pool, bt, sl, out, lse, **args)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


def _identical(outs, what):
    (o0, l0), (o1, l1) = outs
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), f"{what}: LSEs differ"


@pytest.mark.parametrize("layout", ["slices", "separate", "head_major"])
@pytest.mark.parametrize("case", [
    dict(kv="bf16", q_len=1, heads=16, page_size=64, lens=(1, 100, 257)),
    dict(kv="bf16", q_len=4, heads=128, page_size=64, lens=(4, 67, 300)),
    dict(kv="bf16", q_len=3, heads=40, page_size=32, lens=(2, 3, 97)),
    dict(kv="fp8", q_len=2, heads=32, page_size=64, lens=(0, 70, 131)),
])
def test_small_identical_and_vs_oracle(layout, case):
    inp = P.small(seed=300, **case)
    outs = _both(inp, layout)
    _identical(outs, f"{case} {layout}")
    ro, rl = oracle.default().decode(inp)
    G.compare(outs[1][0].float().cpu().numpy(), outs[1][1].cpu().numpy(), ro, rl, fp8=case["kv"] == "fp8",
              what=f"{case} {layout}")


@pytest.mark.parametrize("name", ["deepseek_decode", "mtp_verify"])
def test_full_size_head_major_identical(name):
    inp = generate(name)
    _identical(_both(inp, "head_major"), name)


def test_forced_splits_identical():
    inp = P.small(kv="bf16", q_len=1, heads=128, page_size=32, lens=(5, 300, 1000), seed=301)
    _identical(_both(inp, "head_major", num_splits=7), "split7")

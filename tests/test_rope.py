"""GPU rotary embedding of the rope parts vs the CPU oracle, through the C ABI:
the decode turns each query row's rope part at its token's position before the
scores (mla_decode_qparts_rope), the append turns each new key row's rope part
before storing it (mla_kv_append_rope).  The GPU rotation is bit-exact with the
oracle's, so a decode with rotation equals, byte for byte, a plain decode of the
oracle-rotated query; the appended pool bytes equal the oracle's."""
import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
import oracle
from oracle import rope as R, kv_append as KA
import oracle_pins as P
from mla_synth import generate, rope_cache, decode_positions
import gpu_util as G


def _decode_pair(inp, is_neox, layout="separate", positions=None, **kw):
    """(decode with in-kernel rotation, plain decode of the oracle-rotated query), both on the GPU."""
    B, ql, H, _ = inp.q.shape
    pos = decode_positions(inp) if positions is None else positions
    cache = rope_cache(int(inp.max_seq_len) + 8)
    q, pool, bt, sl = G.to_device(inp)
    args = dict(max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale, k_scale=inp.k_scale,
                min_work_units=inp.workload.min_work_units, **kw)
    out1 = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse1 = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda")
    T = B * ql
    if layout == "separate":
        qn, qr = q[..., :512].reshape(T, H, 512).contiguous(), q[..., 512:].reshape(T, H, 64).contiguous()
    else:   # head-major latent part, padded rope head stride
        qn = q[..., :512].reshape(T, H, 512).transpose(0, 1).contiguous().transpose(0, 1)
        buf = torch.zeros((T, H, 128), dtype=q.dtype, device="cuda")
        buf[..., :64] = q[..., 512:].reshape(T, H, 64)
        qr = buf[..., :64]
    mla.mla_decode_qparts(
        qn, qr, pool, bt, sl, out1, lse1,
        positions=torch.from_numpy(np.ascontiguousarray(pos.reshape(-1), dtype=np.int64)).cuda(),
        cos_sin_cache=torch.from_numpy(cache).cuda(), is_neox=is_neox, **args)
    clamped = np.clip(pos, 0, cache.shape[0] - 1)
    rq = R.rotate_query(inp.q, clamped, cache, is_neox)
    inp_r = dataclasses.replace(inp, q=rq)
    out2 = torch.full_like(out1, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    q2 = torch.from_numpy(rq.view(np.int16)).view(torch.bfloat16).cuda()
    mla.mla_decode(q2, pool, bt, sl, out2, lse2, **args)
    torch.cuda.synchronize()
    return (out1, lse1), (out2, lse2), inp_r


def _identical(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: LSEs differ"


@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("case", [
    dict(kv="bf16", q_len=1, heads=16, page_size=64, lens=(1, 100, 257)),
    dict(kv="bf16", q_len=3, heads=128, page_size=32, lens=(3, 67, 300)),
    dict(kv="fp8", q_len=2, heads=32, page_size=64, lens=(0, 70, 131)),
])
@pytest.mark.parametrize("layout", ["separate", "head_major"])
def test_decode_rotation_vs_oracle(is_neox, case, layout):
    inp = P.small(seed=400, **case)
    a, b, inp_r = _decode_pair(inp, is_neox, layout)
    _identical(a, b, f"{case} neox={is_neox} {layout}")
    ro, rl = oracle.default().decode(inp_r)
    G.compare(a[0].float().cpu().numpy(), a[1].cpu().numpy(), ro, rl, fp8=case["kv"] == "fp8",
              what=f"{case} neox={is_neox}")


def test_decode_positions_clamped():
    inp = P.small(kv="bf16", q_len=2, heads=16, page_size=64, lens=(10, 90), seed=401)
    pos = np.array([[-7, 3], [5, 10 ** 9]], dtype=np.int64)
    a, b, _ = _decode_pair(inp, True, positions=pos)
    _identical(a, b, "clamped positions")


@pytest.mark.parametrize("is_neox", [True, False])
def test_decode_full_size(is_neox):
    inp = generate("deepseek_decode")
    a, b, _ = _decode_pair(inp, is_neox)
    _identical(a, b, f"deepseek neox={is_neox}")


@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_rotation_vs_oracle(is_neox, kv):
    rng = np.random.default_rng(410 + is_neox + 2 * (kv == "fp8"))
    T, N, P_ = 300, 12, 64
    pool = rng.integers(0, 256, size=(N, P_, 576), dtype=np.uint8) if kv == "fp8" else \
        rng.integers(0, 1 << 16, size=(N, P_, 576), dtype=np.uint16)
    x = rng.standard_normal((T, 576)).astype(np.float32) * 2
    rows = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    locs = rng.permutation(N * P_)[:T].astype(np.int64)
    locs[5] = -1
    pos = rng.integers(-3, 5000, size=T).astype(np.int64)
    cache = rope_cache(4096)
    rot = rows.copy()
    rot[:, 512:] = R.rotate(rows[:, 512:], np.clip(pos, 0, 4095), cache, is_neox)
    want = KA.kv_append(pool, rot[:, :512], rot[:, 512:], locs, k_scale=0.75)
    dev_pool = torch.from_numpy(pool).view(torch.float8_e4m3fn).cuda() if kv == "fp8" else \
        torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()
    r = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda()
    mla.mla_kv_append(r[:, :512], r[:, 512:], torch.from_numpy(locs).cuda(), dev_pool, k_scale=0.75,
                      positions=torch.from_numpy(pos).cuda(), cos_sin_cache=torch.from_numpy(cache).cuda(),
                      is_neox=is_neox)
    torch.cuda.synchronize()
    got = dev_pool.view(torch.uint8 if kv == "fp8" else torch.int16).cpu().numpy().view(pool.dtype)
    assert got.tobytes() == want.tobytes()

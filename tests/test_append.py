"""GPU KV-cache append vs the CPU oracle (through the C ABI), bit-exact.

The stored pool bytes must equal the oracle's: a copy for a bf16 pool, the
e4m3fn codes of x / k_scale for an fp8 pool (every bf16 input pattern is
swept), rows at their flat slots, out-of-range slots skipped, every other
slot untouched."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_mla_decode_06_amd as mla
from oracle import kv_append as KA
from mla_synth import Workload, generate, WORKLOADS
from test_oracle_append import decode_step_rows


def _pool_to_dev(pool):
    if pool.dtype == np.uint8:
        return torch.from_numpy(pool).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()


def gpu_append(pool, rows, locs, k_scale=1.0, layout="strided"):
    """pool: host [N, P, 576] uint16/uint8; rows: host [T, 576] bf16 bits.
    layout "strided": k_nope and k_rope are the two slices of one [T, 576]
    tensor; "separate": two contiguous tensors."""
    dev_pool = _pool_to_dev(pool)
    r = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).view(torch.bfloat16).cuda()
    if layout == "strided":
        nope, rope = r[:, :512], r[:, 512:]
    else:
        nope, rope = r[:, :512].contiguous(), r[:, 512:].contiguous()
    loc = torch.from_numpy(np.asarray(locs, dtype=np.int64)).cuda()
    mla.mla_kv_append(nope, rope, loc, dev_pool, k_scale=k_scale)
    torch.cuda.synchronize()
    out = dev_pool.view(torch.uint8) if pool.dtype == np.uint8 else dev_pool.view(torch.int16)
    return out.cpu().numpy().view(pool.dtype)


def _all_bf16_rows():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    T = -(-bits.size // 576)
    rows = np.zeros(T * 576, dtype=np.uint16)
    rows[:bits.size] = bits
    return rows.reshape(T, 576)


@pytest.mark.parametrize("k_scale", [1.0, 0.5, 0.37109375, 3.0])
def test_fp8_every_bf16_pattern(k_scale):
    rows = _all_bf16_rows()
    rng = np.random.default_rng(60)
    N, P = 4, 64
    pool = rng.integers(0, 256, size=(N, P, 576), dtype=np.uint8)
    locs = rng.permutation(N * P)[:rows.shape[0]]
    want = KA.kv_append(pool, rows[:, :512], rows[:, 512:], locs, k_scale=k_scale)
    got = gpu_append(pool, rows, locs, k_scale)
    if got.tobytes() != want.tobytes():
        bad = np.argwhere(got != want)[:8]
        raise AssertionError(f"k_scale {k_scale}: {int((got != want).sum())} bytes differ, first at "
                             f"{bad.tolist()}: got {[int(got[tuple(i)]) for i in bad]}, "
                             f"want {[int(want[tuple(i)]) for i in bad]}")


def test_bf16_every_pattern_copied():
    rows = _all_bf16_rows()
    rng = np.random.default_rng(61)
    N, P = 8, 32
    pool = rng.integers(0, 1 << 16, size=(N, P, 576), dtype=np.uint16)
    locs = rng.permutation(N * P)[:rows.shape[0]]
    want = KA.kv_append(pool, rows[:, :512], rows[:, 512:], locs)
    assert gpu_append(pool, rows, locs).tobytes() == want.tobytes()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [32, 64])
@pytest.mark.parametrize("T", [1, 7, 300])
@pytest.mark.parametrize("layout", ["strided", "separate"])
def test_scatter(kv, P, T, layout):
    rng = np.random.default_rng(1000 * T + P + (kv == "fp8"))
    N = -(-T // P) + 3
    if kv == "fp8":
        pool = rng.integers(0, 256, size=(N, P, 576), dtype=np.uint8)
    else:
        pool = rng.integers(0, 1 << 16, size=(N, P, 576), dtype=np.uint16)
    x = rng.standard_normal((T, 576)).astype(np.float32) * 3
    rows = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    locs = rng.permutation(N * P)[:T].astype(np.int64)
    if T > 2:
        locs[1], locs[2] = -1, N * P      # skipped
    want = KA.kv_append(pool, rows[:, :512], rows[:, 512:], locs, k_scale=0.75)
    got = gpu_append(pool, rows, locs, 0.75, layout)
    assert got.tobytes() == want.tobytes()


def _newest_rows_case(name):
    inp = generate(name)
    rows, locs = decode_step_rows(inp)
    return inp, rows, locs


@pytest.mark.parametrize("name", ["deepseek_decode", "mtp_verify", "long_context"])
def test_decode_step_append_rebuilds_pool(name):
    """At the full decode shapes: blank the slots of every request's newest
    q_len tokens, append those rows on the GPU: the pool is the generated one
    again, byte for byte."""
    inp, rows, locs = _newest_rows_case(name)
    assert rows.shape[0] == inp.batch * inp.q_len
    blank = inp.pool.copy()
    P = inp.page_size
    blank[locs // P, locs % P] = 0x7FC0
    got = gpu_append(blank, rows, locs)
    assert got.tobytes() == inp.pool.tobytes()


def test_decode_step_append_fp8_full_size():
    """The fp8 workload's shape: B new rows (seeded bf16 N(0,1) values) into
    the newest slots of the generated fp8 pool, k_scale 0.5."""
    inp = generate("fp8_kv")
    P = inp.page_size
    locs = np.array([int(inp.block_table[b, (int(L) - 1) // P]) * P + (int(L) - 1) % P
                     for b, L in enumerate(inp.seq_lens)], dtype=np.int64)
    x = np.random.default_rng(62).standard_normal((inp.batch, 576)).astype(np.float32)
    rows = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    want = KA.kv_append(inp.pool, rows[:, :512], rows[:, 512:], locs, k_scale=inp.k_scale)
    got = gpu_append(inp.pool, rows, locs, inp.k_scale)
    assert got.tobytes() == want.tobytes()


def test_append_then_decode_reads_new_rows():
    """The decode after an append sees the appended rows: appending the newest
    rows into a blanked pool and decoding gives the same bytes as decoding
    the generated pool."""
    inp, rows, locs = _newest_rows_case("tiny")
    q, pool, bt, sl = (torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).cuda(),
                       _pool_to_dev(inp.pool), torch.from_numpy(inp.block_table).cuda(),
                       torch.from_numpy(inp.seq_lens).cuda())
    P = inp.page_size
    blank = inp.pool.copy()
    blank[locs // P, locs % P] = 0
    pool2 = _pool_to_dev(blank)
    r = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda()
    mla.mla_kv_append(r[:, :512], r[:, 512:], torch.from_numpy(locs).cuda(), pool2)
    outs = []
    for pl in (pool, pool2):
        out = torch.empty((inp.batch, inp.q_len, inp.heads, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((inp.batch, inp.q_len, inp.heads), dtype=torch.float32, device="cuda")
        mla.mla_decode(q, pl, bt, sl, out, lse, max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def test_large_append():
    """A prefill-sized append: 12000 rows scattered over a 500-page pool."""
    rng = np.random.default_rng(63)
    N, P, T = 500, 32, 12000
    pool = np.zeros((N, P, 576), dtype=np.uint8)
    rows = rng.integers(0, 1 << 16, size=(T, 576), dtype=np.uint16) & 0xBFFF   # finite values
    locs = rng.permutation(N * P)[:T].astype(np.int64)
    want = KA.kv_append(pool, rows[:, :512], rows[:, 512:], locs, k_scale=2.0)
    assert gpu_append(pool, rows, locs, 2.0).tobytes() == want.tobytes()

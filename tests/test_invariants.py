"""GPU invariances and bit-exact properties of the decode (through the C ABI)."""
import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle
import oracle_pins as P
import paged_mla_decode_06_amd as mla
from mla_synth import generate, permute_pages, repack, poison_unused, gather_rows
import gpu_util as G


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("page", [32, 64])
def test_gather_bit_exact(orc, kv, page):
    inp = P.small(kv=kv, page_size=page, lens=(1, 63, 64, 65, 700), heads=4, seed=41)
    q, pool, bt, sl = G.to_device(inp)
    p = mla.params_for(q, pool, bt, inp.max_seq_len, inp.softmax_scale, inp.k_scale)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        dst = torch.zeros((max(L, 1), 576), dtype=pool.dtype, device="cuda")
        mla.mla_gather_kv(p, pool, bt, sl, b, dst)
        torch.cuda.synchronize()
        got = dst[:L].cpu().view(torch.uint8 if kv == "fp8" else torch.int16).numpy()
        want = orc.gather_bytes(inp, b, L)
        assert got.tobytes() == want.tobytes() == gather_rows(inp, b).tobytes()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_single_token_is_the_row(kv):
    """One visible token: the output is that latent row exactly."""
    inp = P.small(kv=kv, lens=(1, 1, 1), heads=128, page_size=64, seed=42)
    o, l = G.run(inp)
    for b in range(inp.batch):
        stored = gather_rows(inp, b)[0]
        if kv == "fp8":
            from oracle import brute
            row = brute.e4m3fn_codes_to_f64(stored)[:512] * inp.k_scale
        else:
            row = (stored[:512].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(o[b, 0], np.broadcast_to(row, (inp.heads, 512))), f"request {b}"


def test_empty_rows():
    inp = P.small(q_len=3, lens=(0, 1, 2, 3, 40), heads=16, seed=43)
    o, l = G.run(inp)
    for b, L in enumerate(inp.seq_lens):
        for j in range(3):
            if int(L) - 3 + 1 + j <= 0:
                assert np.all(o[b, j] == 0) and np.all(np.isneginf(l[b, j]))
            else:
                assert np.all(np.isfinite(l[b, j]))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_page_permutation_bit_exact(kv):
    inp = P.small(kv=kv, lens=(1, 100, 257, 1000), heads=128, seed=44)
    o1, l1 = G.run(inp)
    o2, l2 = G.run(permute_pages(inp, seed=3))
    assert o1.tobytes() == o2.tobytes() and l1.tobytes() == l2.tobytes()


def test_page_size_bit_exact():
    inp = P.small(lens=(1, 100, 257, 1000), heads=128, page_size=64, seed=45)
    o1, l1 = G.run(inp)
    o2, l2 = G.run(repack(inp, 32, seed=4))
    assert o1.tobytes() == o2.tobytes() and l1.tobytes() == l2.tobytes()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_poison_never_read(kv):
    """NaN in every pool slot no request reads and garbage in unused
    block-table entries leave the output bit-identical."""
    inp = P.small(kv=kv, q_len=2, lens=(2, 33, 64, 150, 1000), heads=64, seed=46)
    o1, l1 = G.run(inp)
    dirty = dataclasses.replace(inp, pool=inp.pool.copy(), block_table=inp.block_table.copy())
    poison_unused(dirty)
    dirty.block_table[dirty.block_table < 0] = -1
    o2, l2 = G.run(dirty)
    dirty.block_table[inp.block_table < 0] = 1 << 30
    o3, l3 = G.run(dirty)
    assert o1.tobytes() == o2.tobytes() == o3.tobytes()
    assert l1.tobytes() == l2.tobytes() == l3.tobytes()


@pytest.mark.parametrize("S", [1, 2, 3, 7, 64])
def test_split_count_sweep(orc, S):
    inp = P.small(lens=(1, 333, 2048, 4000), heads=128, seed=47)
    ro, rl = orc.decode(inp)
    o, l = G.run(inp, num_splits=S)
    G.compare(o, l, ro, rl, what=f"splits={S}")
    o2, l2 = G.run(inp, num_splits=S)
    assert o.tobytes() == o2.tobytes() and l.tobytes() == l2.tobytes(), "not deterministic"


# above 256 / nrb groups the launch folds several plan groups into each workgroup
@pytest.mark.parametrize("units", [1, 3, 17, 256, 1000, 4000])
def test_balanced_grid_sweep(orc, units):
    inp = P.small(q_len=2, lens=(2, 333, 2048, 4000), heads=64, seed=48)
    ro, rl = orc.decode(inp)
    o, l = G.run(inp, min_work_units=units)
    G.compare(o, l, ro, rl, what=f"units={units}")


def test_mtp_equals_expanded_single_token():
    inp = P.small(q_len=4, lens=(4, 9, 300, 1000), heads=128, seed=49)
    o, l = G.run(inp)
    B, ql = inp.batch, inp.q_len
    exp_L = np.maximum(np.repeat(inp.seq_lens, ql) - ql + 1 + np.tile(np.arange(ql), B), 0).astype(np.int32)
    w = dataclasses.replace(inp.workload, batch=B * ql, q_len=1)
    single = dataclasses.replace(inp, workload=w, q=inp.q.reshape(B * ql, 1, inp.heads, -1),
                                 block_table=np.repeat(inp.block_table, ql, axis=0), seq_lens=exp_L)
    o1, l1 = G.run(single)
    G.compare(o1.reshape(o.shape), l1.reshape(l.shape), o.astype(np.float64), l.astype(np.float64),
              what="mtp vs expanded")


def test_fp8_equals_bf16_on_dequantised_pool():
    from oracle import brute
    import mla_synth
    f8 = P.small(kv="fp8", lens=(3, 45, 90, 700), heads=128, seed=50, k_scale=0.5)
    vals = brute.e4m3fn_codes_to_f64(f8.pool) * 0.5
    bits = mla_synth.f32_to_bf16_bits(vals.astype(np.float32))
    w = dataclasses.replace(f8.workload, kv="bf16", k_scale=1.0)
    b16 = dataclasses.replace(f8, workload=w, pool=bits, k_scale=1.0)
    o1, l1 = G.run(f8)
    o2, l2 = G.run(b16)
    G.compare(o1, l1, o2.astype(np.float64), l2.astype(np.float64), fp8=True, what="fp8 vs dequantised bf16")


# min_work_units 1000 and 3000: more groups than the CUs hold, so the plan
# kernel runs folded (several plan groups per workgroup) as the decode does
@pytest.mark.parametrize("mode", [dict(), dict(num_splits=5), dict(min_work_units=37), dict(min_work_units=1000),
                                  dict(min_work_units=3000)])
def test_device_plan_equals_host_plan(mode):
    L = np.array([0, 1, 31, 32, 33, 500, 4096, 77], dtype=np.int32)
    p = mla.make_params(len(L), 2, 128, 64, 1000, 64, 4096, mla.MLA_KV_BF16, 0.07, 1.0,
                        mode.get("num_splits", 0), mode.get("min_work_units", 0), 0)
    pieces, grid = mla.mla_plan_host(p, L)
    dev_pieces, counts = mla.mla_plan_device(p, torch.from_numpy(L).cuda(), grid, 64)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    dp = dev_pieces.cpu().numpy()
    got = np.concatenate([dp[g, :counts[g]] for g in range(grid)]) if counts.sum() else np.zeros((0, 6), np.int32)
    assert counts.max() <= 64
    assert np.array_equal(got, pieces)

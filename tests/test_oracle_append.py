"""Pins for the KV-append oracle (CPU only): the e4m3fn encoder against
torch's own float8 cast and the closed forms of the format, and the scatter
against the seeded generator's pool layout and the pinned C oracle's gather."""
import numpy as np
import pytest

import oracle
from oracle import kv_append as KA
from mla_synth import Workload, generate

torch = pytest.importorskip("torch")


def _torch_codes(x):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _sweep():
    """Every bf16 value as float32, divided by a few scales, plus random
    float32 values and values a hair either side of every rounding midpoint."""
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    with np.errstate(over="ignore"):
        parts = [allbf / np.float32(s) for s in (1.0, 0.5, 0.37109375, 3.0)]
    rng = np.random.default_rng(0)
    parts.append(rng.standard_normal(200000).astype(np.float32) * np.float32(40.0))
    vals = KA._POS_VALUES
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    parts += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), -mids]
    with np.errstate(over="ignore"):
        x = np.concatenate(parts).astype(np.float32)
    return np.clip(x, -448.0, 448.0).astype(np.float32)


def test_encoder_matches_torch_cast():
    x = _sweep()
    assert KA.e4m3fn_encode(x).tobytes() == _torch_codes(x).tobytes()


def test_encoder_closed_forms():
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([KA.e4m3fn_value(c) for c in codes], dtype=np.float32)
    assert np.array_equal(KA.e4m3fn_encode(vals), np.array(codes, dtype=np.uint8)), "value -> code round trip"
    e = KA.e4m3fn_encode
    assert e([448.0])[0] == 0x7E and e([-448.0])[0] == 0xFE
    assert e([1e30])[0] == 0x7E and e([-np.inf])[0] == 0xFE and e([np.inf])[0] == 0x7E   # saturation
    assert e([0.0])[0] == 0x00 and e([-0.0])[0] == 0x80
    assert e([np.nan])[0] == 0x7F and e([-np.nan])[0] == 0x7F
    assert e([2.0 ** -9])[0] == 0x01                       # smallest subnormal
    assert e([2.0 ** -10])[0] == 0x00                      # tie between 0 and 2^-9: even code 0
    assert e([1.5 * 2.0 ** -10])[0] == 0x01
    assert e([1.0])[0] == 0x38 and e([1.0625])[0] == 0x38   # 1 + 1/16: tie between 0x38 and 0x39 -> even
    assert e([1.1875])[0] == 0x3A                          # 1 + 3/16: tie between 0x39 and 0x3A -> even
    assert e([240.0])[0] == 0x77 and e([232.0])[0] == 0x76  # 232 = tie 224 | 240 -> even (0x76)


def test_encoder_relative_error_bound():
    """Inside the normal range the stored value is within half a unit of the
    3-bit mantissa, |v - x| <= 2^-4 |x|; below it within half the subnormal
    step, |v - x| <= 2^-10."""
    rng = np.random.default_rng(1)
    x = (rng.uniform(-1, 1, 100000) * np.exp2(rng.uniform(-12, 8.7, 100000))).astype(np.float32)
    c = KA.e4m3fn_encode(x)
    v = np.array([KA.e4m3fn_value(int(k)) for k in c])
    err = np.abs(v - x.astype(np.float64))
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10)


@pytest.mark.parametrize("mutant", ["ties_away", "truncate"])
def test_encoder_pin_catches_planted_mistakes(mutant):
    vals = KA._POS_VALUES

    def bad(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        a = np.minimum(np.abs(x), 448.0)
        if mutant == "truncate":
            idx = np.searchsorted(vals, a, side="right") - 1
        else:
            d = np.abs(a[:, None] - vals[None, :])
            idx = len(vals) - 1 - np.argmin(d[:, ::-1], axis=1)   # the larger value on a tie
        return np.where(np.signbit(x), idx | 0x80, idx).astype(np.uint8)

    x = _sweep()
    assert bad(x).tobytes() != _torch_codes(x).tobytes()


def decode_step_rows(inp):
    """The rows of each request's last q_len tokens (the tokens a decode step
    appends), read through the pinned C oracle's gather, and their flat slots
    page * page_size + slot (the meaning of out_cache_loc)."""
    orc = oracle.default()
    rows, locs = [], []
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        if L == 0:
            continue
        t0 = max(L - inp.q_len, 0)
        rows.append(orc.gather_bytes(inp, b, L)[t0:L])
        for t in range(t0, L):
            locs.append(int(inp.block_table[b, t // inp.page_size]) * inp.page_size + t % inp.page_size)
    return np.concatenate(rows), np.array(locs, dtype=np.int64)


def test_scatter_rebuilds_generator_pool():
    """Blank the slots of each request's newest tokens in a generated bf16 pool,
    append those rows again: the pool is bit-identical to the generated one."""
    w = Workload(name="append", batch=5, q_len=3, heads=16, page_size=32, kv="bf16", seed=21,
                 lens=("fixed", [3, 40, 64, 65, 130]))
    inp = generate(w)
    rows, locs = decode_step_rows(inp)
    blank = inp.pool.copy()
    P = inp.page_size
    for s in locs:
        blank[s // P, s % P] = 0x7FC0
    got = KA.kv_append(blank, rows[:, :512], rows[:, 512:], locs)
    assert got.tobytes() == inp.pool.tobytes()


def test_scatter_skips_out_of_range_and_keeps_other_slots():
    rng = np.random.default_rng(3)
    N, P = 6, 64
    pool = rng.integers(0, 1 << 16, size=(N, P, 576), dtype=np.uint16)
    rows = rng.integers(0, 1 << 16, size=(4, 576), dtype=np.uint16)
    locs = np.array([-1, N * P, 5, N * P - 1], dtype=np.int64)
    got = KA.kv_append(pool, rows[:, :512], rows[:, 512:], locs)
    want = pool.copy()
    want[0, 5] = rows[2]
    want[N - 1, P - 1] = rows[3]
    assert got.tobytes() == want.tobytes()


def test_fp8_append_dequantises_close_to_input():
    """An fp8 append stores codes whose dequantised values (code * k_scale, by
    the pinned C oracle's decoder) are within half a mantissa unit of the
    bf16 input."""
    rng = np.random.default_rng(4)
    T, N, P, ks = 50, 4, 32, 0.5
    x = rng.standard_normal((T, 576)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)            # truncation: any bf16 values will do
    pool = np.zeros((N, P, 576), dtype=np.uint8)
    locs = rng.permutation(N * P)[:T].astype(np.int64)
    got = KA.kv_append(pool, bits[:, :512], bits[:, 512:], locs, k_scale=ks)
    orc = oracle.default()
    xb = KA.bf16_bits_to_f32(bits).astype(np.float64)
    for i in range(0, T, 7):
        s = int(locs[i])
        deq = np.array([orc.e4m3fn(int(c)) for c in got[s // P, s % P]]) * ks
        small = np.abs(xb[i]) < 2.0 ** -6 * ks
        assert np.all(np.abs(deq - xb[i])[~small] <= 2.0 ** -4 * np.abs(xb[i])[~small])
        assert np.all(np.abs(deq - xb[i])[small] <= 2.0 ** -10 * ks)

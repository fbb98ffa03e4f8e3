"""The seeded input generator: storage rounding, layout and determinism (no GPU)."""
import numpy as np
import torch

import mla_synth
from mla_synth import generate, WORKLOADS


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]     # ties to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mla_synth.f32_to_bf16_bits(x), ref)


def test_e4m3_codes_are_nearest():
    from oracle import brute   # decoder only, to read the codes back
    x = np.random.default_rng(1).standard_normal(50000).astype(np.float32) * 40
    x[:3] = [1000.0, -1000.0, 0.0]
    codes = mla_synth.f32_to_e4m3fn_codes(x)
    vals = brute.e4m3fn_codes_to_f64(codes)
    table = brute.e4m3fn_codes_to_f64(np.arange(256, dtype=np.uint8))
    finite = table[np.isfinite(table)]
    xc = np.clip(x.astype(np.float64), -448, 448)
    best = np.min(np.abs(xc[:, None] - finite[None, :]), axis=1)
    assert np.array_equal(np.abs(xc - vals), best)
    assert vals[0] == 448 and vals[1] == -448


def test_tiny_layout():
    inp = generate("tiny")
    assert inp.q.shape == (2, 1, 16, 576) and inp.q.dtype == np.uint16
    assert inp.pool.shape == (16, 64, 576)
    assert inp.block_table.shape == (2, 5)
    assert list(inp.block_table[0, 2:]) == [-1, -1, -1]
    used = np.concatenate([inp.block_table[0, :2], inp.block_table[1, :5]])
    assert len(set(used.tolist())) == 7 and used.min() >= 0 and used.max() < 16


def test_deterministic():
    a = generate("tiny")
    b = generate("tiny")
    assert a.q.tobytes() == b.q.tobytes() and a.pool.tobytes() == b.pool.tobytes()
    c = generate("tiny", seed=77)
    assert c.q.tobytes() != a.q.tobytes()


def test_workload_shapes():
    import math
    w = WORKLOADS["long_context"]
    rng = np.random.default_rng(w.seed)
    L = mla_synth.gen.draw_seq_lens(w, rng)
    assert L[0] == 32768 and L.min() >= 1 and L.max() <= 32768 and w.page_size == 32
    for name, lo, hi in [("deepseek_decode", 1024, 4096), ("mtp_verify", 2048, 8192), ("fp8_kv", 512, 4096)]:
        w = WORKLOADS[name]
        L = mla_synth.gen.draw_seq_lens(w, np.random.default_rng(w.seed))
        assert L.min() >= lo and L.max() <= hi and L.shape == (w.batch,)
    assert abs(mla_synth.SOFTMAX_SCALE_F32 - 1 / math.sqrt(192)) < 1e-8
    assert np.float32(mla_synth.SOFTMAX_SCALE_F32).view(np.uint32) == 0x3D93CD3A


def test_poison_marks_only_unread_slots():
    inp = generate("tiny", poison=True)
    for b in range(2):
        rows = mla_synth.gather_rows(inp, b)
        assert not np.any(rows == mla_synth.BF16_NAN)
    assert np.count_nonzero(inp.pool == mla_synth.BF16_NAN) > 0

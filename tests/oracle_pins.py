"""Pins for the CPU oracle: checks against what the mathematics and the pages
fix, independent of the oracle's own code.

Each pin takes an ``oracle.Oracle`` (the default build, or a build with a
planted mistake) and raises AssertionError when the oracle disagrees.  The
pins are chosen so that a plausible slip anywhere in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong log base) fails at
least one of them; ``test_oracle_mutants.py`` checks exactly that.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import mla_synth
from mla_synth import Workload, generate, permute_pages, repack, poison_unused
from oracle import brute

REL = 1e-12


def small(kv="bf16", q_len=1, heads=8, page_size=32, lens=(1, 31, 32, 33, 100), seed=11, k_scale=None,
          num_pages=None) -> mla_synth.Inputs:
    w = Workload(name="pin", batch=len(lens), q_len=q_len, heads=heads, page_size=page_size, kv=kv, seed=seed,
                 lens=("fixed", list(lens)), num_pages=num_pages,
                 k_scale=(0.5 if kv == "fp8" else 1.0) if k_scale is None else k_scale)
    return generate(w)


def _close(a, b, rel=REL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        scale = max(1.0, float(np.max(np.abs(b[fin]))))
        err = float(np.max(np.abs(a[fin] - b[fin])))
        assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:.0e} * {scale:.3g}"


def _identical(a, b, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape and a.tobytes() == b.tobytes(), f"{what}: not bit-identical"


# ---------------------------------------------------------------- decoders
def pin_bf16_decoder(orc):
    """Every non-NaN bf16 code decodes to torch's bfloat16 -> float64 value."""
    import torch
    codes = np.arange(0, 1 << 16, 7, dtype=np.uint16)   # a spread including subnormals, inf, +-0
    codes = np.concatenate([codes, np.array([0x0000, 0x8000, 0x0001, 0x7F7F, 0x7F80, 0xFF80, 0x3F80], np.uint16)])
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16(int(c)) for c in codes])
    keep = ~np.isnan(ref)
    assert np.array_equal(got[keep], ref[keep]), "bf16 decode differs from torch"
    assert np.isnan(got[~keep]).all()


def pin_fp8_decoder(orc):
    """All 256 e4m3fn codes decode to torch's float8_e4m3fn -> float64 value (NaN at S.1111.111)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3fn(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    keep = ~np.isnan(ref)
    assert np.array_equal(got[keep], ref[keep]), "e4m3fn decode differs from torch"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ---------------------------------------------------------------- brute force
def pin_brute(orc, inp):
    """Paged fp64 loop == dense numpy attention over the gathered rows."""
    o1, l1 = orc.decode(inp)
    o2, l2 = brute.decode(inp)
    _close(o1, o2, what="out vs brute")
    _close(l1, l2, what="lse vs brute")


def brute_cases():
    return [
        small(),
        small(page_size=64, lens=(64, 65, 300), heads=16, seed=12),
        small(q_len=4, heads=4, lens=(4, 5, 37, 130), seed=13),
        small(q_len=2, heads=3, page_size=64, lens=(2, 64, 129), seed=14),
        small(kv="fp8", lens=(1, 40, 97), heads=4, seed=15),
        small(kv="fp8", q_len=3, heads=2, page_size=64, lens=(3, 70, 200), k_scale=0.37, seed=16),
    ]


# ---------------------------------------------------------------- invariances
def pin_page_permutation(orc, inp):
    """Shuffling pool pages and mapping the block table through the shuffle changes nothing."""
    o1, l1 = orc.decode(inp)
    o2, l2 = orc.decode(permute_pages(inp, seed=99))
    _identical(o1, o2, "out after page permutation")
    _identical(l1, l2, "lse after page permutation")


def pin_page_size(orc, inp):
    """The same token rows packed with page size 32 and 64 give the same result."""
    other = 64 if inp.page_size == 32 else 32
    o1, l1 = orc.decode(inp)
    o2, l2 = orc.decode(repack(inp, other, seed=7))
    _identical(o1, o2, "out after repacking")
    _identical(l1, l2, "lse after repacking")


def pin_split_merge(orc, inp):
    """Attention over contiguous token ranges, merged by log-sum-exp, equals attention over the whole range."""
    rng = np.random.default_rng(5)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        rows = orc.gather_rows(inp, b, L)
        for j in range(inp.q_len):
            n = L - inp.q_len + 1 + j
            if n <= 0:
                continue
            h = int(rng.integers(inp.heads))
            qrow = inp.q[b, j, h]
            full_o, full_l = orc.attend(qrow, rows, 0, n, inp.softmax_scale)
            for S in sorted({1, 2, 3, 7, n}):
                if S > n:
                    continue
                cuts = np.linspace(0, n, S + 1).round().astype(int)
                parts = [orc.attend(qrow, rows, int(a), int(c), inp.softmax_scale) for a, c in zip(cuts[:-1], cuts[1:])]
                o, l = orc.merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
                _close(o, full_o, what=f"merge S={S}")
                _close(l, full_l, what=f"merge lse S={S}")
    # all-empty parts merge to o = 0, lse = -inf
    o, l = orc.merge(np.zeros((3, 8)), np.full(3, -np.inf))
    assert np.all(o == 0) and l == -np.inf


def pin_key_order(orc, inp):
    """With one query token, the order in which a request's rows sit in its pages does not matter."""
    assert inp.q_len == 1
    rng = np.random.default_rng(3)
    shuffled = dataclasses.replace(inp, pool=inp.pool.copy())
    P = inp.page_size
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        rows = mla_synth.gather_rows(inp, b)
        perm = rng.permutation(L)
        t = np.arange(L)
        shuffled.pool[inp.block_table[b, t // P], t % P] = rows[perm]
    o1, l1 = orc.decode(inp)
    o2, l2 = orc.decode(shuffled)
    _close(o1, o2, what="out after key shuffle")
    _close(l1, l2, what="lse after key shuffle")


def pin_poison(orc, inp):
    """NaN in every slot no request reads and garbage in unused block-table entries change nothing."""
    clean = dataclasses.replace(inp, pool=inp.pool.copy(), block_table=inp.block_table.copy())
    dirty = dataclasses.replace(inp, pool=inp.pool.copy(), block_table=inp.block_table.copy())
    poison_unused(dirty)
    dirty.block_table[dirty.block_table < 0] = 1 << 30
    o1, l1 = orc.decode(clean)
    o2, l2 = orc.decode(dirty)
    _identical(o1, o2, "out with poison")
    _identical(l1, l2, "lse with poison")


def pin_mtp_expansion(orc, inp):
    """Multi-token causal decode == one single-token decode per query token j with
    seq_len L - q_len + 1 + j and the same block-table row (the draft catch-up
    expansion of "tokenspeed trtllm_mla.py", TRTLLMMLABackend.forward_decode)."""
    ql = inp.q_len
    assert ql > 1
    o, l = orc.decode(inp)
    B = inp.batch
    exp_q = inp.q.reshape(B * ql, 1, inp.heads, -1)
    exp_bt = np.repeat(inp.block_table, ql, axis=0)
    exp_L = (np.repeat(inp.seq_lens, ql) - ql + 1 + np.tile(np.arange(ql), B)).astype(np.int32)
    exp_L = np.maximum(exp_L, 0)
    w = dataclasses.replace(inp.workload, batch=B * ql, q_len=1)
    single = dataclasses.replace(inp, workload=w, q=exp_q, block_table=exp_bt, seq_lens=exp_L)
    o1, l1 = orc.decode(single)
    _identical(o1.reshape(o.shape), o, "mtp vs expanded out")
    _identical(l1.reshape(l.shape), l, "mtp vs expanded lse")


# ---------------------------------------------------------------- closed forms
def _decoded_q(inp, b, j, h):
    return brute.bf16_bits_to_f64(inp.q[b, j, h])


def pin_single_token(orc, kv="bf16"):
    """One visible token: the output is that token's latent row exactly and
    lse is its scaled score."""
    inp = small(kv=kv, lens=(1, 1), heads=4, seed=21)
    o, l = orc.decode(inp)
    for b in range(inp.batch):
        stored = mla_synth.gather_rows(inp, b)[0]
        row = (brute.e4m3fn_codes_to_f64(stored) * inp.k_scale) if inp.kv_fp8 else brute.bf16_bits_to_f64(stored)
        for h in range(inp.heads):
            assert np.array_equal(o[b, 0, h], row[:512]), "single token: out != row"
            s = inp.softmax_scale * float(np.dot(_decoded_q(inp, b, 0, h), row))
            _close(l[b, 0, h], s, what="single token lse")


def pin_zero_query(orc):
    """Q = 0 gives uniform weights: out = mean of the latent rows, lse = ln n."""
    inp = small(lens=(1, 7, 64, 100), heads=2, seed=22)
    inp.q[...] = 0
    o, l = orc.decode(inp)
    for b in range(inp.batch):
        rows = brute.bf16_bits_to_f64(mla_synth.gather_rows(inp, b))
        n = rows.shape[0]
        for h in range(inp.heads):
            _close(o[b, 0, h], rows[:, :512].mean(axis=0), what="zero query out")
            _close(l[b, 0, h], np.log(n), what="zero query lse")


def pin_equal_rows(orc):
    """All visible rows equal r: out = r[:512], lse = scale*q.r + ln n."""
    inp = small(lens=(5, 70), heads=3, seed=23)
    P = inp.page_size
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        t = np.arange(L)
        r = inp.pool[inp.block_table[b, 0], 0].copy()
        inp.pool[inp.block_table[b, t // P], t % P] = r
    o, l = orc.decode(inp)
    for b in range(inp.batch):
        r = brute.bf16_bits_to_f64(mla_synth.gather_rows(inp, b)[0])
        n = int(inp.seq_lens[b])
        for h in range(inp.heads):
            _close(o[b, 0, h], r[:512], what="equal rows out")
            s = inp.softmax_scale * float(np.dot(_decoded_q(inp, b, 0, h), r))
            _close(l[b, 0, h], s + np.log(n), what="equal rows lse")


def pin_empty(orc):
    """No visible token: out = 0 and lse = -inf (seq_len 0, or a query token
    that precedes every cached row)."""
    inp = small(q_len=3, lens=(0, 1, 2, 3), heads=2, seed=24)
    o, l = orc.decode(inp)
    for b, L in enumerate(inp.seq_lens):
        for j in range(3):
            n = int(L) - 3 + 1 + j
            if n <= 0:
                assert np.all(o[b, j] == 0) and np.all(l[b, j] == -np.inf), (b, j)
            else:
                assert np.all(np.isfinite(l[b, j])), (b, j)


def pin_fp8_equals_dequantised_bf16(orc):
    """An fp8 pool with k_scale == the bf16 pool holding code*k_scale exactly
    (every e4m3fn value times 0.5 is a bf16 value) with no scale."""
    f8 = small(kv="fp8", lens=(3, 45, 90), heads=4, seed=25, k_scale=0.5)
    vals = brute.e4m3fn_codes_to_f64(f8.pool) * 0.5
    bits = mla_synth.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(brute.bf16_bits_to_f64(bits), vals)        # exact
    w = dataclasses.replace(f8.workload, kv="bf16", k_scale=1.0)
    b16 = dataclasses.replace(f8, workload=w, pool=bits, k_scale=1.0)
    o1, l1 = orc.decode(f8)
    o2, l2 = orc.decode(b16)
    _identical(o1, o2, "fp8 vs dequantised bf16 out")
    _identical(l1, l2, "fp8 vs dequantised bf16 lse")


def pin_gather_bytes(orc, inp):
    """Byte gather through the block table == numpy fancy-index gather."""
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        _identical(orc.gather_bytes(inp, b, L), mla_synth.gather_rows(inp, b), f"gather b={b}")


def pin_decode_rows(orc, inp):
    """Selected-row decode == the same rows of the full decode."""
    o, l = orc.decode(inp)
    sel = [(b, j, h) for b in range(inp.batch) for j in range(inp.q_len) for h in (0, inp.heads - 1)]
    so, sl = orc.decode_rows(inp, sel)
    for k, (b, j, h) in enumerate(sel):
        _identical(so[k], o[b, j, h], "decode_rows out")
        _identical(sl[k], l[b, j, h], "decode_rows lse")


def all_pins(orc):
    """Run every pin on small inputs; returns the list of (name, error) failures."""
    fails = []

    def run(name, fn, *a):
        try:
            fn(orc, *a)
        except (AssertionError, ValueError) as e:
            fails.append((name, str(e)[:200]))

    run("bf16_decoder", pin_bf16_decoder)
    run("fp8_decoder", pin_fp8_decoder)
    for i, inp in enumerate(brute_cases()):
        run(f"brute[{i}]", pin_brute, inp)
    base = small(lens=(1, 33, 64, 150), heads=4, seed=31)
    run("page_permutation", pin_page_permutation, base)
    run("page_size", pin_page_size, base)
    run("split_merge", pin_split_merge, small(q_len=2, lens=(2, 40, 150), heads=3, seed=32))
    run("key_order", pin_key_order, base)
    run("poison", pin_poison, small(q_len=2, lens=(2, 40, 150), heads=3, seed=33))
    run("mtp_expansion", pin_mtp_expansion, small(q_len=4, lens=(4, 9, 100), heads=3, seed=34))
    run("single_token_bf16", pin_single_token, "bf16")
    run("single_token_fp8", pin_single_token, "fp8")
    run("zero_query", pin_zero_query)
    run("equal_rows", pin_equal_rows)
    run("empty", pin_empty)
    run("fp8_vs_bf16", pin_fp8_equals_dequantised_bf16)
    run("gather_bytes", pin_gather_bytes, base)
    run("decode_rows", pin_decode_rows, small(q_len=2, lens=(2, 40), heads=3, seed=35))
    return fails

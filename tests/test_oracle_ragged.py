"""Pins for the ragged-decode oracle (CPU only): it reduces to the uniform
oracle when every request has the same query length, agrees with the dense
brute force per request, and each of its rows equals a single-token decode
at the row's visible length."""
import numpy as np

import oracle
from oracle import ragged as RG
import oracle_pins as P
from mla_synth import generate, ragged


def test_uniform_lengths_reduce_to_uniform_oracle():
    inp = P.small(q_len=3, heads=8, page_size=32, lens=(3, 40, 64, 65), seed=41)
    rg = ragged(inp, q_lens=[3, 3, 3, 3])
    o, l = RG.decode(oracle.default(), rg)
    ro, rl = oracle.default().decode(inp)
    assert np.array_equal(o, ro.reshape(-1, 8, 512)) and np.array_equal(l, rl.reshape(-1, 8))


def test_matches_dense_brute_force():
    for kv in ("bf16", "fp8"):
        inp = P.small(kv=kv, q_len=4, heads=4, page_size=32, lens=(1, 5, 33, 70, 2), seed=42)
        rg = ragged(inp, q_lens=[1, 4, 0, 3, 2])
        o, l = RG.decode(oracle.default(), rg)
        bo, bl = RG.decode(None, rg, dense=True)
        P._close(o, bo, what=f"{kv} out")
        P._close(l, bl, what=f"{kv} lse")


def test_rows_equal_single_token_decodes():
    """Row (b, j) sees exactly the first L_b - q_b + 1 + j tokens: it equals a
    one-token decode of request b with that many cached tokens."""
    inp = P.small(q_len=4, heads=4, page_size=64, lens=(4, 9, 70), seed=43)
    rg = ragged(inp, q_lens=[2, 4, 1])
    o, l = RG.decode(oracle.default(), rg)
    orc = oracle.default()
    for b in range(3):
        qb, L = int(rg.q_lens[b]), int(inp.seq_lens[b])
        for j in range(qb):
            t = int(rg.qo_indptr[b]) + j
            v = RG.request_view(rg, b)
            v.q = rg.q[t:t + 1][None]
            v.q_len = 1
            v.seq_lens = np.array([L - qb + 1 + j], dtype=np.int32)
            so, sl = orc.decode(v)
            assert np.array_equal(o[t], so[0, 0]) and np.array_equal(l[t], sl[0, 0]), (b, j)


def test_empty_requests_and_sampled_rows():
    inp = P.small(q_len=2, heads=4, page_size=32, lens=(0, 10, 40), seed=44)
    rg = ragged(inp, q_lens=[0, 2, 1])
    assert rg.total_q == 3 and list(rg.qo_indptr) == [0, 0, 2, 3]
    o, l = RG.decode(oracle.default(), rg)
    sel = [(2, 3), (0, 1), (1, 0)]
    so, sl = RG.decode_rows(oracle.default(), rg, sel)
    for i, (t, h) in enumerate(sel):
        assert np.array_equal(so[i], o[t, h]) and sl[i] == l[t, h]


def test_generator_packs_first_q_b_tokens():
    inp = generate("tiny")
    rg = ragged(inp, q_lens=[1, 1])
    assert np.array_equal(rg.q[0], inp.q[0, 0]) and np.array_equal(rg.q[1], inp.q[1, 0])

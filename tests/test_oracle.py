"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def test_bf16_decoder(orc):
    P.pin_bf16_decoder(orc)


def test_fp8_decoder(orc):
    P.pin_fp8_decoder(orc)


@pytest.mark.parametrize("case", range(len(P.brute_cases())))
def test_brute_force(orc, case):
    P.pin_brute(orc, P.brute_cases()[case])


@pytest.mark.parametrize("page_size", [32, 64])
def test_page_permutation(orc, page_size):
    P.pin_page_permutation(orc, P.small(page_size=page_size, lens=(1, 33, 64, 150), heads=4, seed=31))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_page_size(orc, kv):
    P.pin_page_size(orc, P.small(kv=kv, lens=(1, 33, 64, 150), heads=4, seed=31))


def test_split_merge(orc):
    P.pin_split_merge(orc, P.small(q_len=2, lens=(2, 40, 150), heads=3, seed=32))


def test_key_order(orc):
    P.pin_key_order(orc, P.small(lens=(1, 33, 64, 150), heads=4, seed=31))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_poison(orc, kv):
    P.pin_poison(orc, P.small(kv=kv, q_len=2, lens=(2, 40, 150), heads=3, seed=33))


@pytest.mark.parametrize("q_len", [2, 4])
def test_mtp_expansion(orc, q_len):
    P.pin_mtp_expansion(orc, P.small(q_len=q_len, lens=(q_len, 9, 100), heads=3, seed=34))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_single_token(orc, kv):
    P.pin_single_token(orc, kv)


def test_zero_query(orc):
    P.pin_zero_query(orc)


def test_equal_rows(orc):
    P.pin_equal_rows(orc)


def test_empty_rows(orc):
    P.pin_empty(orc)


def test_fp8_equals_dequantised_bf16(orc):
    P.pin_fp8_equals_dequantised_bf16(orc)


def test_gather_bytes(orc):
    P.pin_gather_bytes(orc, P.small(lens=(1, 33, 64, 150), heads=4, seed=31))
    P.pin_gather_bytes(orc, P.small(kv="fp8", lens=(5, 64), heads=2, seed=36))


def test_decode_rows(orc):
    P.pin_decode_rows(orc, P.small(q_len=2, lens=(2, 40), heads=3, seed=35))


def test_bad_page_raises(orc):
    inp = P.small(lens=(40,), heads=2, seed=37)
    inp.block_table[0, 1] = inp.num_pages      # read by token 32..39
    with pytest.raises(ValueError):
        orc.decode(inp)


def test_tiny_workload_brute(orc):
    """The 2-request, 16-head tiny workload itself against dense brute force."""
    from mla_synth import generate
    inp = generate("tiny")
    assert list(inp.seq_lens) == [100, 257] and inp.num_pages == 16 and inp.block_table.shape == (2, 5)
    P.pin_brute(orc, inp)


def test_brute_decoders_match_torch():
    """The dense checker's own decoders agree with torch's dtype casts."""
    import torch
    from oracle import brute
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = brute.e4m3fn_codes_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])
    b = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = brute.bf16_bits_to_f64(b)
    keep = ~np.isnan(ref)
    assert np.array_equal(got[keep], ref[keep])

"""Pins of the oracle's fp8 query (oracle/query_fp8.py) against torch's float8
cast (the cast the pages apply to the query of their fp8 decode) and closed
forms of the format."""
import numpy as np
import pytest

from oracle.query_fp8 import quantize_query

torch = pytest.importorskip("torch")


def _f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_every_bf16_pattern_against_torch_cast():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = _f32(bits)
    got = _f32(quantize_query(bits))
    fin = np.isfinite(x)
    inr = fin & (np.abs(x) <= 448)
    ref = torch.from_numpy(x[inr].copy()).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    # in range: torch's cast, sign of zero included
    assert np.array_equal(got[inr].view(np.uint32), ref.view(np.uint32))
    # beyond +-448 (and the infinities): saturated
    big = ~np.isnan(x) & (np.abs(x) > 448)
    assert np.array_equal(got[big], np.where(x[big] > 0, 448.0, -448.0).astype(np.float32))
    assert np.isnan(got[np.isnan(x)]).all()


def test_closed_forms():
    # ties to the even mantissa: 1 + 1/16 lies halfway between 1 and 1.125
    # (mantissas 0 and 1), 1 + 3/16 between 1.125 and 1.25 (1 and 2)
    cases = {1.0625: 1.0, 1.1875: 1.25, -1.0625: -1.0, 2 ** -9: 2 ** -9, 2 ** -10: 0.0, 3 * 2 ** -10: 2 ** -8,
             240.0: 240.0, 248.0: 256.0, 464.0: 448.0, 0.3: 0.3125, -17.0: -16.0}
    x = np.array(list(cases), dtype=np.float32)
    got = _f32(quantize_query(_bits(x)))
    assert np.array_equal(got, np.array(list(cases.values()), dtype=np.float32)), (x, got)


def test_idempotent():
    rng = np.random.default_rng(5)
    bits = _bits(rng.standard_normal(20000).astype(np.float32) * 30)
    once = quantize_query(bits)
    assert np.array_equal(quantize_query(once), once)
    assert quantize_query(bits.reshape(100, 200)).shape == (100, 200)

"""Pins for the rotary-embedding oracle (CPU only): the complex-number closed
form of a rotation, the identity at angle 0, the relation between the
interleaved and the rotate-half layouts, and planted mistakes that the closed
form catches."""
import numpy as np
import pytest

from oracle import rope as R
from mla_synth import rope_cache


def _bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32) * 2
    return R._f32_to_bf16(x)


def _complex_ref(bits, pos, cache, is_neox):
    """y = (x1 + i x2) * exp(i theta) in fp64, with cos/sin from the cache."""
    x = R._bf16_to_f32(bits).astype(np.float64)
    cs = cache[np.asarray(pos)].astype(np.float64)
    a, b = R.pair_index(is_neox)
    z = (x[..., a] + 1j * x[..., b]) * (cs[..., :32] + 1j * cs[..., 32:])
    y = np.empty_like(x)
    y[..., a], y[..., b] = z.real, z.imag
    return y


def _check_close(got_bits, ref, what):
    got = R._bf16_to_f32(got_bits).astype(np.float64)
    # bf16 rounding of the result (2^-9 relative) plus float32 rounding of the
    # two products and the sum, relative to the operands' size
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * (1 + np.abs(ref))
    assert np.all(np.abs(got - ref) <= bound), f"{what}: max err {np.max(np.abs(got - ref)):.3e}"


@pytest.mark.parametrize("is_neox", [True, False])
def test_matches_complex_rotation(is_neox):
    rng = np.random.default_rng(1)
    cache = rope_cache(4096)
    bits = _bits(rng, (300, 64))
    pos = rng.integers(0, 4096, size=300)
    _check_close(R.rotate(bits, pos, cache, is_neox), _complex_ref(bits, pos, cache, is_neox), f"neox={is_neox}")


@pytest.mark.parametrize("is_neox", [True, False])
def test_position_zero_is_identity(is_neox):
    rng = np.random.default_rng(2)
    bits = _bits(rng, (50, 64))
    out = R.rotate(bits, np.zeros(50, dtype=np.int64), rope_cache(4), is_neox)
    assert np.array_equal(out, bits)


def test_interleaved_is_rotate_half_on_deinterleaved():
    rng = np.random.default_rng(3)
    cache = rope_cache(1000)
    bits = _bits(rng, (200, 64))
    pos = rng.integers(0, 1000, size=200)
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])   # interleaved -> halves
    inv = np.argsort(perm)
    a = R.rotate(bits, pos, cache, is_neox=False)
    b = R.rotate(bits[:, perm], pos, cache, is_neox=True)[:, inv]
    assert np.array_equal(a, b)


def test_query_rotation_touches_only_the_rope_part():
    rng = np.random.default_rng(4)
    q = _bits(rng, (2, 3, 4, 576))
    pos = np.array([[5, 6, 7], [0, 1, 2]])
    out = R.rotate_query(q, pos, rope_cache(16), True)
    assert np.array_equal(out[..., :512], q[..., :512])
    assert np.array_equal(out[1, 0, :, 512:], q[1, 0, :, 512:])          # position 0
    assert not np.array_equal(out[0, 0, :, 512:], q[0, 0, :, 512:])


@pytest.mark.parametrize("mutant", ["sin_sign", "cos_sin_swapped", "wrong_pairs"])
def test_closed_form_catches_planted_mistakes(mutant):
    rng = np.random.default_rng(5)
    cache = rope_cache(512)
    bits = _bits(rng, (100, 64))
    pos = rng.integers(1, 512, size=100)
    if mutant == "sin_sign":
        bad = R.rotate(bits, pos, np.concatenate([cache[:, :32], -cache[:, 32:]], axis=1), True)
    elif mutant == "cos_sin_swapped":
        bad = R.rotate(bits, pos, np.concatenate([cache[:, 32:], cache[:, :32]], axis=1), True)
    else:
        bad = R.rotate(bits, pos, cache, False)
    with pytest.raises(AssertionError):
        _check_close(bad, _complex_ref(bits, pos, cache, True), mutant)

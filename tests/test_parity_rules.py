"""CPU tests of the comparison rules the GPU parity tests apply (tests/parity.py): the
single-rounding rule for reconstructed keys accepts exactly the nearest-even rounding of the
oracle's value, and a neighbouring value only where the oracle's value lies within the
stated band of the midpoint between the two."""
import numpy as np
import pytest

import oracle
from kv_cache_vector_windowed_amd import synth
from parity import check_rounded_once


def _values(seed, n=4000):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * np.exp(rng.uniform(-5, 5, n))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_rounding_passes(dtype):
    ref = _values(1)
    mag = np.abs(ref) * 2
    if dtype == "bf16":
        got = synth.bf16_bits_to_f32(oracle.round_bf16(ref))
    else:
        got = ref.astype(np.float32)
    assert check_rounded_once(got, ref, mag, dtype) == 0


def _neighbour(got32, dtype, step):
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(got32).astype(np.int64) + step
        return synth.bf16_bits_to_f32(bits.astype(np.uint16))
    return (got32.view(np.uint32).astype(np.int64) + step).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_neighbour_only_inside_the_band(dtype):
    ref = _values(2, 64)
    ref = np.where(ref > 0, ref, -ref)  # positive: bits + 1 is the next value up
    exact = synth.bf16_bits_to_f32(oracle.round_bf16(ref)) if dtype == "bf16" else ref.astype(np.float32)
    up = _neighbour(exact, dtype, 1)
    mid = 0.5 * (exact.astype(np.float64) + up.astype(np.float64))
    mag = 2 * np.abs(ref)
    pmax = 2 ** 17
    delta = (pmax * 2.0 ** -51 + 2.0 ** -50) * mag
    # a value just below the midpoint (inside the band) may come out as either neighbour
    inside = mid - 0.5 * delta
    assert check_rounded_once(up, inside, mag, dtype, pmax) == inside.size
    assert check_rounded_once(exact, inside, mag, dtype, pmax) == 0
    # well away from the midpoint only the nearest value passes
    outside = mid - 4 * delta
    with pytest.raises(AssertionError):
        check_rounded_once(up, outside, mag, dtype, pmax)
    # two units away never passes
    with pytest.raises(AssertionError):
        check_rounded_once(_neighbour(exact, dtype, 2), inside, mag, dtype, pmax)


def test_nan_rows_must_match():
    ref = np.array([1.0, np.nan, 3.0])
    got = np.array([1.0, np.nan, 3.0], np.float32)
    assert check_rounded_once(got, ref, np.ones(3), "f32") == 0
    with pytest.raises(AssertionError):
        check_rounded_once(np.array([1.0, 2.0, 3.0], np.float32), ref, np.ones(3), "f32")

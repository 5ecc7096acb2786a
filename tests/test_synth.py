"""The seeded input generators: deterministic, the stated shapes and distributions."""
import numpy as np

from kv_cache_vector_windowed_amd import synth


def test_deterministic_and_distinct_streams():
    a = synth.draw(0, 0, 100, 1)
    b = synth.draw(0, 0, 100, 1)
    c = synth.draw(0, 0, 100, 2)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert not np.array_equal(synth.draw(0, 1, 100, 1), a)


def test_variances_and_outliers():
    s, outl = synth.key_distribution(1, 3)
    assert s.min() >= 0.1 and s.max() <= 10.0 and len(set(outl.tolist())) == 4
    x = synth.draw(1, 3, 20000, 1).astype(np.float64)
    var = x.var(axis=0)
    expect = s.copy()
    expect[outl] *= 400.0
    np.testing.assert_allclose(var, expect, rtol=0.05)


def test_bf16_keys_are_exact():
    k = synth.keys(0, 2, 64, "bf16")
    assert k.values.dtype == np.float32 and k.bits.dtype == np.uint16
    assert np.array_equal(synth.f32_to_bf16_bits(k.values), k.bits)
    assert np.array_equal(k.values.view(np.uint32) & 0xFFFF, np.zeros(k.values.shape, np.uint32))


def test_queries_covariance():
    q = synth.queries(0, 1, 20000, d=16)[0].astype(np.float64)
    a = synth.rng(0, 0, 3).standard_normal((16, 16)) / 4.0
    np.testing.assert_allclose(q.T @ q / len(q), a @ a.T, atol=0.05)


def test_workload_table():
    w = synth.WORKLOADS
    assert [w[k].cfg for k in ("tiny", "layer", "decode", "encode_stress", "long_context")] == \
        [0, 1, 2, 3, 4]
    assert w["tiny"].n == 4096 and w["encode_stress"].c == 4096 and w["decode"].batch == 32

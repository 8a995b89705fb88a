"""Pins for the oracle's random numbers.

Philox4x32-10 is the counter-based generator of Salmon et al. (SC'11).  The oracle's
implementation is checked against rocRAND's public host-callable Philox4x32-10 engine, built
here from its installed header and run as a separate program (nothing is copied from it).
The uniform / Gumbel conversions are checked by their ranges and distributions.
"""
import numpy as np
from scipy import stats

import oracle

# the rocRAND Philox fixture (rocrand_pin) lives in conftest.py


def test_philox_matches_rocrand(rocrand_pin):
    rng = np.random.default_rng(1)
    n = 3000
    ctrs = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    # small counters, the shapes the method uses, and the all-zero / all-ones corners
    ctrs[:500, 1:] = rng.integers(0, 64, size=(500, 3), dtype=np.uint64).astype(np.uint32)
    ctrs[0] = 0
    ctrs[1] = 0xFFFFFFFF
    keys = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    keys[0] = 0
    keys[1] = 0xFFFFFFFF
    ref = rocrand_pin(keys, ctrs)
    got = np.stack([oracle.philox(c[None], k)[0] for c, k in zip(ctrs[:200], keys[:200])])
    np.testing.assert_array_equal(got, ref[:200])
    # batch path, one key
    key = keys[7]
    ref_b = rocrand_pin(np.repeat(key[None], n, 0), ctrs)
    np.testing.assert_array_equal(oracle.philox(ctrs, key), ref_b)


def test_uniform_uses_documented_counter_layout(rocrand_pin):
    """uniform(seed, req, pos, v, stream) = ((w >> 8) + 0.5) 2^-24 with w = word v&3 of the
    block at counter (v>>2, pos, req, stream), key = (seed low, seed high)."""
    rng = np.random.default_rng(2)
    seed = 0xD5A0000000000006
    n = 400
    req = rng.integers(0, 600, n)
    pos = rng.integers(0, 17, n)
    v = rng.integers(0, 262144, n)
    stream = 2
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64).astype(np.uint32)
    ctrs = np.stack([v >> 2, pos, req, np.full(n, stream)], 1).astype(np.uint32)
    words = rocrand_pin(np.repeat(key[None], n, 0), ctrs)[np.arange(n), v & 3]
    expect = ((words >> 8).astype(np.float64) + 0.5) / 2.0**24
    got = oracle.uniform(seed, req, pos, v, stream)
    np.testing.assert_array_equal(got, expect)


def test_uniform_open_interval_and_flat():
    u = oracle.uniform(123, 7, 3, np.arange(1_000_000), 0)
    assert u.min() > 0.0 and u.max() < 1.0
    counts, _ = np.histogram(u, bins=100, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-4
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / len(u))


def test_neighbouring_indices_are_independent():
    """Four consecutive v share one Philox block but use different words; consecutive
    draws must be uncorrelated and distinct."""
    u = oracle.uniform(99, 5, 0, np.arange(400_000), 0)
    assert np.all(u[0::4] != u[1::4])
    r = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(r) < 4 / np.sqrt(len(u))
    # streams, positions and request keys select different blocks
    a = oracle.uniform(99, 5, 0, np.arange(4096), 0)
    for other in (oracle.uniform(99, 5, 0, np.arange(4096), 1),
                  oracle.uniform(99, 5, 1, np.arange(4096), 0),
                  oracle.uniform(99, 6, 0, np.arange(4096), 0),
                  oracle.uniform(100, 5, 0, np.arange(4096), 0)):
        assert abs(np.corrcoef(a, other)[0, 1]) < 0.1
        assert np.mean(a == other) < 0.01


def test_gumbel_distribution():
    """-log(-log u) is standard Gumbel: compare against scipy's CDF."""
    import ctypes
    L = oracle.lib()
    g = np.array([L.oracle_gumbel(ctypes.c_uint64(11), 3, 1, v, 0) for v in range(60_000)])
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-4
    assert abs(g.mean() - np.euler_gamma) < 4 * np.pi / np.sqrt(6) / np.sqrt(len(g))

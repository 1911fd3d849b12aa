"""The oracle's codebook (closed-form Gaussian quantile table, seeded order).

Pins: the inverse normal CDF against the Python standard library's NormalDist and
scipy's ndtri (a different algorithm), and against the defining property
Phi(Phi^-1(p)) = p; SplitMix64 against its published test vectors; the table is an
exactly antisymmetric set of quantiles placed in a permuted order; the product grid
for V = 2.
"""
import statistics

import numpy as np
import pytest
from scipy import special


def test_inv_normal_cdf_against_library(oracle_lib):
    nd = statistics.NormalDist()
    ps = np.concatenate([np.linspace(1e-6, 1 - 1e-6, 4001), [1e-300, 1e-100, 1e-20, 1e-10,
                                                              0.0249, 0.0251, 0.5, 0.9751]])
    for p in ps:
        x = oracle_lib.inv_normal_cdf(p)
        assert abs(x - nd.inv_cdf(p)) <= 4e-15 * max(1.0, abs(x)), p
        y = special.ndtri(p)
        assert abs(x - y) <= 1e-13 * max(1.0, abs(x)), p
        if 1e-12 < p < 1 - 1e-12:
            assert abs(special.ndtr(x) - p) <= 1e-14 * max(p, 1e-3)


def test_splitmix64_published_vectors(oracle_lib):
    # reference outputs of SplitMix64 (Steele, Lea, Flood 2014; Vigna's splitmix64.c)
    assert oracle_lib.splitmix64_stream(0, 1)[0] == 0xE220A8397B1DCDAF
    assert oracle_lib.splitmix64_stream(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


@pytest.mark.parametrize("L", [1, 2, 8, 12, 16])
def test_codebook_v1_is_shuffled_quantiles(oracle_lib, L):
    nd = statistics.NormalDist()
    N = 1 << L
    C = oracle_lib.make_codebook(L, 1, 3000 + L)
    assert C.shape == (N, 1) and C.dtype == np.float32
    srt = np.sort(C[:, 0])
    expect = np.array([nd.inv_cdf((j + 0.5) / N) for j in range(N)], dtype=np.float64)
    assert np.array_equal(srt, expect.astype(np.float32))
    assert np.array_equal(srt, -srt[::-1])               # exact antisymmetry
    if L >= 8:
        # really shuffled, deterministic per seed, different across seeds
        assert not np.array_equal(C[:, 0], srt)
        assert np.array_equal(C, oracle_lib.make_codebook(L, 1, 3000 + L))
        assert not np.array_equal(C, oracle_lib.make_codebook(L, 1, 1 + L))


def test_codebook_shuffle_definition(oracle_lib):
    # Fisher-Yates from the top, j = SplitMix64 output mod (i+1), on a 4-entry table
    L, seed = 2, 42
    base = np.array([statistics.NormalDist().inv_cdf((j + 0.5) / 4) for j in range(4)],
                    dtype=np.float64).astype(np.float32)
    stream = oracle_lib.splitmix64_stream(seed, 3)
    a = list(base)
    for step, i in enumerate(range(3, 0, -1)):
        j = stream[step] % (i + 1)
        a[i], a[j] = a[j], a[i]
    C = oracle_lib.make_codebook(L, 1, seed)
    assert np.array_equal(C[:, 0], np.array(a, dtype=np.float32))


def test_codebook_v2_product_grid(oracle_lib):
    L, V = 16, 2
    C = oracle_lib.make_codebook(L, V, 3004)
    g = np.sort(oracle_lib.make_codebook(8, 1, 0)[:, 0])
    assert C.shape == (1 << 16, 2)
    # every row is a point of the 256 x 256 grid, and every grid point occurs once
    ia = np.searchsorted(g, C[:, 0])
    ib = np.searchsorted(g, C[:, 1])
    assert np.array_equal(g[ia], C[:, 0]) and np.array_equal(g[ib], C[:, 1])
    assert np.unique(ia * 256 + ib).size == 1 << 16

"""Pins for the soft-trellis (BCJR) oracle, oracle.bcjr_block.

B1  brute force: for tiny trellises every path is enumerated (tests/brute_force.py),
    scored in float64, and Z = sum exp(-J/tau) and the expectation of the emitted
    values are formed directly; the forward-backward result must agree.
B2  tau -> 0: the soft codeword tends to the Viterbi reconstruction and -tau log Z to
    the Viterbi cost (the BCJR-QAT abstract: the hard code is recovered as the
    temperature goes to 0).
B3  tau -> infinity: every path equally likely; with a free start every state is then
    equally likely at every step, so the soft codeword is the column mean of the
    codebook and log Z = log(number of paths) = (L - kV + kV n) log 2.
B4  derivative: d(-tau log Z)/dw_i = 2 d_i (w_i - soft_i) (the gradient of the free
    energy is the expected gradient of J), checked by central differences.
B5  scaling d and tau by the same factor changes nothing.
"""
import numpy as np
import pytest

import brute_force as bf


def _brute(w, d, C, L, k, V, T, tau):
    _, states = bf.enumerate_paths(w, d, C, L, k, V, T)
    n = T // V
    Cd = np.asarray(C, dtype=np.float64).reshape(1 << L, V)
    vals = Cd[states[:, 1:]].reshape(states.shape[0], n * V)      # [P, T]
    dd = np.ones(T) if d is None else np.asarray(d, dtype=np.float64)
    J = ((np.asarray(w, dtype=np.float64)[None, :] - vals) ** 2 * dd[None, :]).sum(axis=1)
    m = (-J / tau).max()
    p = np.exp(-J / tau - m)
    Z = p.sum()
    return (p[:, None] * vals).sum(axis=0) / Z, m + np.log(Z)


@pytest.mark.parametrize("L,k,V,T,tau", [(4, 1, 1, 4, 0.3), (5, 2, 1, 3, 0.05),
                                         (4, 1, 2, 4, 1.0), (6, 2, 1, 4, 0.02),
                                         (3, 1, 1, 6, 0.5), (6, 3, 1, 3, 0.2)])
def test_brute_force(oracle_lib, L, k, V, T, tau):
    import oracle
    rng = np.random.default_rng(L * 10 + T)
    C = oracle.make_codebook(L, V, 5 + L)
    for weighted in (False, True):
        w = rng.standard_normal(T).astype(np.float32)
        d = np.exp(rng.standard_normal(T)).astype(np.float32) if weighted else None
        soft, logz = oracle.bcjr_block(w, d, C, L, k, V, T, tau)
        bsoft, blogz = _brute(w, d, C, L, k, V, T, tau)
        assert np.allclose(soft, bsoft, rtol=1e-10, atol=1e-12)
        assert abs(logz - blogz) <= 1e-10 * max(1.0, abs(blogz))


@pytest.mark.parametrize("L,k,V,T", [(8, 2, 1, 32), (6, 1, 2, 12), (10, 3, 1, 24)])
def test_zero_temperature_is_viterbi(oracle_lib, L, k, V, T):
    import oracle
    rng = np.random.default_rng(L + T)
    C = oracle.make_codebook(L, V, 21)
    checked = 0
    for _ in range(6):
        w = rng.standard_normal(T).astype(np.float32)
        bits, s0, cost = oracle.encode_block(w, None, C, L, k, V, T)
        best, second = oracle.two_best_block(w, None, C, L, k, V, T)
        gap = float(second) - float(best)
        if gap < 1e-4:
            continue
        tau = gap / 80.0
        hard = oracle.decode_block(bits, s0, C, L, k, V, T)
        soft, logz = oracle.bcjr_block(w, None, C, L, k, V, T, tau)
        assert np.allclose(soft, hard, atol=1e-6 * (1 + np.abs(hard).max()))
        assert abs(-tau * logz - float(cost)) <= 1e-5 * float(cost) + 2 * tau
        checked += 1
    assert checked >= 3


@pytest.mark.parametrize("L,k,V,T", [(6, 2, 1, 16), (8, 2, 2, 8)])
def test_infinite_temperature_is_uniform(oracle_lib, L, k, V, T):
    import oracle
    C = oracle.make_codebook(L, V, 2)
    w = np.random.default_rng(0).standard_normal(T).astype(np.float32)
    soft, logz = oracle.bcjr_block(w, None, C, L, k, V, T, 1e12)
    mean = np.tile(C.astype(np.float64).mean(axis=0), T // V)
    assert np.allclose(soft, mean, atol=1e-9)
    kv, n = k * V, T // V
    assert abs(logz - (L - kv + kv * n) * np.log(2.0)) < 1e-6


@pytest.mark.parametrize("L,k,V,T,tau", [(6, 2, 1, 12, 0.1), (8, 2, 2, 8, 0.5)])
def test_free_energy_gradient(oracle_lib, L, k, V, T, tau):
    import oracle
    rng = np.random.default_rng(L * T)
    C = oracle.make_codebook(L, V, 8)
    w = rng.standard_normal(T)
    d = np.exp(0.5 * rng.standard_normal(T))
    soft, _ = oracle.bcjr_block(w, d, C, L, k, V, T, tau)
    h = 1e-6
    for i in range(T):
        wp, wm = w.copy(), w.copy()
        wp[i] += h
        wm[i] -= h
        fp = -tau * oracle.bcjr_block(wp, d, C, L, k, V, T, tau)[1]
        fm = -tau * oracle.bcjr_block(wm, d, C, L, k, V, T, tau)[1]
        fd = (fp - fm) / (2 * h)
        assert abs(fd - 2 * d[i] * (w[i] - soft[i])) < 1e-6 * (1 + abs(fd)), i


def test_scale_invariance(oracle_lib):
    import oracle
    L, k, V, T = 8, 2, 1, 24
    rng = np.random.default_rng(4)
    C = oracle.make_codebook(L, V, 1)
    w = rng.standard_normal(T)
    d = np.exp(rng.standard_normal(T))
    s1, z1 = oracle.bcjr_block(w, d, C, L, k, V, T, 0.2)
    s2, z2 = oracle.bcjr_block(w, 2 * d, C, L, k, V, T, 0.4)
    assert np.allclose(s1, s2, rtol=1e-12, atol=1e-12) and abs(z1 - z2) < 1e-9 * abs(z1)

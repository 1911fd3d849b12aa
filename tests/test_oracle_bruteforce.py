"""The oracle against exhaustive enumeration of every path (tiny trellises).

O1  oracle cost == brute-force minimum, bitwise
O2  the oracle's own path, scored independently, has exactly the oracle's cost
O3  on dyadic inputs (all arithmetic exact, ties frequent) the oracle's path is the
    optimal path with the smallest tie key (s_n, j_n, ..., j_2): lowest end state,
    then lowest predecessor index at each step going back
O4  the oracle's runner-up equals the second smallest cost of all paths
"""
import itertools

import numpy as np
import pytest

import brute_force as bf


def _cases():
    out = []
    for L in range(2, 7):
        for k in (1, 2, 3):
            for V in (1, 2):
                kv = k * V
                if kv > L:
                    continue
                for T in range(V, 7, V):
                    paths = 2 ** (L - kv + k * T)
                    if paths > 2 ** 15:
                        continue
                    out.append((L, k, V, T))
    return out


CASES = _cases()


def test_fmaf32_matches_libm():
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    b = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    c = (rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))).astype(np.float32)
    got = bf.fmaf32(a, b, c)
    ref = np.array([bf.libm_fmaf(x, y, z) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fmaf32_double_rounding_case():
    # exact a*b + c = 1 + 2^-23 + 2^-24 - 2^-70: rounding the float64 sum (which lands
    # on the float32 midpoint) with ties-to-even would give 1 + 2^-22; the exact value
    # lies below the midpoint, so the correct fmaf is 1 + 2^-23.
    a = np.float32(2.0 ** -24 * (1 + 2.0 ** -23))
    b = np.float32(1 - 2.0 ** -23)
    c = np.float32(1 + 2.0 ** -23)
    naive = np.float32(np.float64(a) * np.float64(b) + np.float64(c))
    assert naive == np.float32(1 + 2.0 ** -22)
    assert bf.fmaf32(a, b, c) == np.float32(1 + 2.0 ** -23)
    assert bf.libm_fmaf(a, b, c) == np.float32(1 + 2.0 ** -23)


def _random_problem(rng, L, k, V, T, weighted, cb_kind):
    w = rng.standard_normal(T).astype(np.float32)
    if cb_kind == "random":
        C = rng.standard_normal((1 << L, V)).astype(np.float32)
    else:
        import oracle
        C = oracle.make_codebook(L, V, int(rng.integers(1 << 30)))
    d = np.exp(rng.standard_normal(T)).astype(np.float32) if weighted else None
    return w, d, C


@pytest.mark.parametrize("L,k,V,T", CASES)
def test_oracle_matches_bruteforce(oracle_lib, L, k, V, T):
    rng = np.random.default_rng(1000 * L + 100 * k + 10 * V + T)
    for trial, (weighted, cb_kind) in enumerate(itertools.product((False, True),
                                                                   ("random", "quantile"))):
        w, d, C = _random_problem(rng, L, k, V, T, weighted, cb_kind)
        bits, s0, cost = oracle_lib.encode_block(w, d, C, L, k, V, T)
        best, second, _, _, costs, states = bf.best_path(w, d, C, L, k, V, T)
        # O1
        assert cost.view(np.uint32) == best.view(np.uint32), (trial, cost, best)
        # O2: locate the oracle's path among the enumerated ones and compare its score
        kv = k * V
        n = T // V
        sel = states[:, 0] == s0
        for t in range(1, n + 1):
            b = 0
            for i in range(kv):
                pos = (t - 1) * kv + i
                b = (b << 1) | ((int(bits[pos // 32]) >> (31 - pos % 32)) & 1)
            sel &= (states[:, t] & ((1 << kv) - 1)) == b
        assert sel.sum() == 1
        assert costs[sel][0].view(np.uint32) == cost.view(np.uint32)
        # O4
        b1, b2 = oracle_lib.two_best_block(w, d, C, L, k, V, T)
        assert b1.view(np.uint32) == best.view(np.uint32)
        assert b2.view(np.uint32) == second.view(np.uint32), (b2, second)


def _dyadic_problem(rng, L, V, T):
    w = (rng.integers(-12, 13, T) / 8.0).astype(np.float32)
    C = (rng.integers(-12, 13, ((1 << L), V)) / 8.0).astype(np.float32)
    d = rng.choice(np.array([0.0, 0.5, 1.0, 2.0], dtype=np.float32), T)
    return w, d, C


@pytest.mark.parametrize("L,k,V,T", CASES)
def test_oracle_tie_rule_dyadic(oracle_lib, L, k, V, T):
    rng = np.random.default_rng(7 + 1000 * L + 100 * k + 10 * V + T)
    for trial in range(3):
        w, d, C = _dyadic_problem(rng, L, V, T)
        if trial == 2:
            d = None
        bits, s0, cost = oracle_lib.encode_block(w, d, C, L, k, V, T)
        best, _, bbits, bs0, costs, _ = bf.best_path(w, d, C, L, k, V, T)
        assert cost == best
        assert s0 == bs0 and np.array_equal(bits, bbits), (trial, bits, bbits, s0, bs0)


@pytest.mark.parametrize("L,k,V,T", [c for c in CASES if c[0] - c[1] * c[2] >= 1][:20])
def test_oracle_fixed_start(oracle_lib, L, k, V, T):
    rng = np.random.default_rng(99 + L * 7 + T)
    w, d, C = _random_problem(rng, L, k, V, T, True, "random")
    kv = k * V
    free_cost = oracle_lib.encode_block(w, d, C, L, k, V, T)[2]
    fixed = []
    for s0 in range(1 << (L - kv)):
        bits, s0_out, cost = oracle_lib.encode_block(w, d, C, L, k, V, T, fixed_s0=s0)
        best = bf.best_path(w, d, C, L, k, V, T, fixed_s0=s0)[0]
        assert s0_out == s0
        assert cost.view(np.uint32) == best.view(np.uint32)
        fixed.append(cost)
    # a free start is the best of all fixed starts
    assert free_cost == min(fixed)


@pytest.mark.parametrize("L,k,V,T", [(4, 1, 1, 5), (5, 2, 1, 4), (6, 2, 2, 4), (6, 3, 1, 3)])
def test_oracle_overflowed_costs(oracle_lib, L, k, V, T):
    """A weight of 1e20 squares past the fp32 range, so every path costs +inf.
    With it first, every comparison of the search is between equal (+inf) costs, so the
    optimum with the smallest tie key -- the all-zero path: end state 0, predecessor 0 at
    every step -- is what the lowest-index rule must return.  With it second, the step-2
    choices still compare finite prefixes; the end state must still be state 0 (the
    lowest index among equal final costs) and the path a valid one of cost +inf."""
    rng = np.random.default_rng(31 + L + T)
    w, d, C = _random_problem(rng, L, k, V, T, True, "quantile")
    w0 = w.copy()
    w0[0] = np.float32(1e20)
    bits, s0, cost = oracle_lib.encode_block(w0, d, C, L, k, V, T)
    best, _, bbits, bs0, costs, _ = bf.best_path(w0, d, C, L, k, V, T)
    assert np.all(np.isinf(costs)) and np.isinf(best) and np.isinf(cost)
    assert s0 == bs0 == 0 and np.array_equal(bits, bbits) and not bits.any()
    w1 = w.copy()
    w1[V] = np.float32(1e20)
    bits, s0, cost = oracle_lib.encode_block(w1, d, C, L, k, V, T)
    assert np.isinf(cost) and s0 < (1 << (L - k * V))
    last_chunk_bits = k * V
    tail = T // V * k * V  # bits in the stream
    assert bf_last_chunk(bits, tail, last_chunk_bits) == 0
    assert np.isinf(oracle_lib.path_cost(w1, d, C, L, k, V, T, bits, s0))


def bf_last_chunk(bits, nbits, kv):
    """Value of the last kv-bit chunk of an MSB-first packed stream of nbits bits."""
    v = 0
    for pos in range(nbits - kv, nbits):
        v = (v << 1) | ((int(bits[pos // 32]) >> (31 - pos % 32)) & 1)
    return v

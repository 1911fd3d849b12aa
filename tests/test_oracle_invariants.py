"""Closed forms and invariants the oracle must satisfy at any size.

T3  memoryless trellis (kV = L): every step chooses freely, so the optimum is the
    per-step best choice (greedy is optimal); one step (T = V): argmin over the table.
T4  uniform weights: d == 1 is bitwise the unweighted search; d == 2^p scales every
    cost exactly by 2^p with identical paths; a non-dyadic uniform d keeps the paths
    except at near-ties.
T5  decode round trip: the decoded path rescored gives the reported cost; a free start
    is the best of all fixed starts.
T6  distortion sanity (not parity): on N(0,1) weights at 2.0547 bits/weight the
    mean squared error lies between the Gaussian rate-distortion bound 2^(-2R) and the
    4-level Lloyd-Max quantizer's error 0.1175.
"""
import numpy as np
import pytest

import brute_force as bf


def _greedy_memoryless(w, d, C, L, k, V, T):
    """kV == L: s_t is b_t; pick, at each step, the lowest state with the smallest
    chained cost."""
    n = T // V
    acc = np.zeros(1, dtype=np.float32)
    states = []
    allst = np.arange(1 << L)
    for t in range(n):
        a = np.repeat(acc, allst.size)
        for v in range(V):
            i = t * V + v
            e = (np.float32(w[i]) - C[allst, v]).astype(np.float32)
            de = e if d is None else (np.float32(d[i]) * e).astype(np.float32)
            a = bf.fmaf32(de, e, a)
        s = int(np.argmin(a))       # first index of the minimum
        states.append(s)
        acc = a[s:s + 1]
    return acc[0], states


@pytest.mark.parametrize("L,k,V,T", [(3, 3, 1, 9), (4, 2, 2, 8), (6, 3, 2, 6), (5, 5, 1, 20),
                                     (8, 4, 2, 16)])
def test_memoryless_is_independent_rounding(oracle_lib, L, k, V, T):
    rng = np.random.default_rng(L * 31 + T)
    for weighted in (False, True):
        w = rng.standard_normal(T).astype(np.float32)
        C = rng.standard_normal((1 << L, V)).astype(np.float32)
        d = np.exp(rng.standard_normal(T)).astype(np.float32) if weighted else None
        bits, s0, cost = oracle_lib.encode_block(w, d, C, L, k, V, T)
        gcost, gstates = _greedy_memoryless(w, d, C, L, k, V, T)
        assert s0 == 0
        assert cost.view(np.uint32) == np.float32(gcost).view(np.uint32)
        dec = oracle_lib.decode_block(bits, s0, C, L, k, V, T)
        assert np.array_equal(dec.reshape(-1, V), C[gstates])


@pytest.mark.parametrize("L,k,V", [(6, 2, 1), (8, 2, 2), (10, 3, 1), (12, 4, 1)])
def test_single_step_is_table_argmin(oracle_lib, L, k, V):
    rng = np.random.default_rng(L)
    T = V
    w = rng.standard_normal(T).astype(np.float32)
    C = rng.standard_normal((1 << L, V)).astype(np.float32)
    d = np.exp(rng.standard_normal(T)).astype(np.float32)
    bits, s0, cost = oracle_lib.encode_block(w, d, C, L, k, V, T)
    a = np.zeros(1 << L, dtype=np.float32)
    for v in range(V):
        e = (w[v] - C[:, v]).astype(np.float32)
        a = bf.fmaf32((d[v] * e).astype(np.float32), e, a)
    s = int(np.argmin(a))
    assert cost == a[s]
    kv = k * V
    assert s0 == s >> kv
    assert int(bits[0]) >> (32 - kv) == s & ((1 << kv) - 1)


@pytest.mark.parametrize("L,k,V,T", [(8, 2, 1, 64), (10, 3, 1, 30), (8, 2, 2, 32),
                                     (12, 2, 1, 48)])
def test_uniform_weights(oracle_lib, L, k, V, T):
    import oracle
    rng = np.random.default_rng(5 + L + T)
    C = oracle.make_codebook(L, V, 77 + L)
    for trial in range(4):
        w = rng.standard_normal(T).astype(np.float32)
        b0, s00, c0 = oracle_lib.encode_block(w, None, C, L, k, V, T)
        b1, s01, c1 = oracle_lib.encode_block(w, np.ones(T, np.float32), C, L, k, V, T)
        assert np.array_equal(b0, b1) and s00 == s01
        assert c0.view(np.uint32) == c1.view(np.uint32)
        for p in (-3, 2):
            bp, s0p, cp = oracle_lib.encode_block(w, np.full(T, 2.0 ** p, np.float32), C,
                                                  L, k, V, T)
            assert np.array_equal(b0, bp) and s00 == s0p
            assert cp == np.float32(c0 * np.float32(2.0 ** p))


def test_uniform_nondyadic_weights_keep_paths(oracle_lib):
    import oracle
    L, k, V, T = 10, 2, 1, 64
    C = oracle.make_codebook(L, V, 5)
    rng = np.random.default_rng(3)
    same = 0
    trials = 40
    for _ in range(trials):
        w = rng.standard_normal(T).astype(np.float32)
        b0, s00, c0 = oracle_lib.encode_block(w, None, C, L, k, V, T)
        b1, s01, c1 = oracle_lib.encode_block(w, np.full(T, 0.7, np.float32), C, L, k, V, T)
        assert abs(float(c1) / float(c0) - 0.7) < 1e-5
        if np.array_equal(b0, b1) and s00 == s01:
            same += 1
        else:
            # only a near-tie may flip: the runner-up is within rounding of the best
            best, second = oracle_lib.two_best_block(w, None, C, L, k, V, T)
            assert (float(second) - float(best)) / float(best) < 1e-5
    assert same >= trials - 2


@pytest.mark.parametrize("L,k,V,T", [(8, 2, 1, 64), (9, 3, 1, 33), (8, 2, 2, 64),
                                     (16, 2, 1, 32), (7, 1, 1, 50)])
def test_decode_roundtrip(oracle_lib, L, k, V, T):
    import oracle
    rng = np.random.default_rng(L * 3 + T)
    C = oracle.make_codebook(L, V, 123)
    w = rng.standard_normal(T).astype(np.float32)
    d = np.exp(rng.standard_normal(T)).astype(np.float32)
    bits, s0, cost = oracle_lib.encode_block(w, d, C, L, k, V, T)
    assert s0 < 1 << (L - k * V)
    rec = oracle_lib.decode_block(bits, s0, C, L, k, V, T)
    # rescore the reconstruction independently of the oracle's chain
    acc = np.float32(0)
    for i in range(T):
        e = np.float32(w[i] - rec[i])
        acc = bf.fmaf32(np.float32(d[i] * e), e, acc)
    assert np.float32(acc).view(np.uint32) == cost.view(np.uint32)
    assert oracle_lib.path_cost(w, d, C, L, k, V, T, bits, s0) == cost
    # unused tail bits of the last word are zero
    nbits = k * T
    if nbits % 32:
        assert int(bits[-1]) & ((1 << (32 - nbits % 32)) - 1) == 0


def test_free_start_is_best_fixed_start(oracle_lib):
    import oracle
    L, k, V, T = 8, 2, 1, 40
    C = oracle.make_codebook(L, V, 9)
    w = np.random.default_rng(4).standard_normal(T).astype(np.float32)
    free = oracle_lib.encode_block(w, None, C, L, k, V, T)
    fixed = [oracle_lib.encode_block(w, None, C, L, k, V, T, fixed_s0=s)[2]
             for s in range(1 << (L - k * V))]
    assert free[2] == min(fixed)
    assert free[1] == int(np.argmin(fixed)) or fixed[free[1]] == free[2]


def test_distortion_sanity_L16(oracle_lib):
    """N(0,1) weights, L=16, k=2, T=256: rate 2 + 14/256 bits per weight."""
    import oracle
    L, k, V, T = 16, 2, 1, 256
    C = oracle.make_codebook(L, V, 3001)
    rng = np.random.default_rng(1)
    W = rng.standard_normal((3, T)).astype(np.float32)
    mse = []
    for r in range(W.shape[0]):
        bits, s0, cost = oracle_lib.encode_block(W[r], None, C, L, k, V, T)
        mse.append(float(cost) / T)
    rate = k + (L - k * V) / T
    m = float(np.mean(mse))
    assert 2.0 ** (-2 * rate) < m < 0.1175, m


def test_decode_gemv_definition(oracle_lib):
    """The decode-then-matvec reference: a unit vector picks a decoded column, and the
    product is linear in x."""
    import oracle
    L, k, V, T, M, N = 10, 2, 1, 32, 5, 96
    rng = np.random.default_rng(21)
    C = oracle.make_codebook(L, V, 4)
    W = rng.standard_normal((M, N)).astype(np.float32)
    bits, s0, _ = oracle.encode_matrix(W, None, C, L, k, V, T)
    What = oracle.decode_matrix(bits, s0, C, M, N, L, k, V, T)
    for j in (0, 31, 32, 95):
        e = np.zeros(N, np.float32)
        e[j] = 1.0
        y, _ = oracle.decode_gemv(bits, s0, C, e, M, N, L, k, V, T)
        assert np.array_equal(y, What[:, j].astype(np.float64))
    x1 = rng.standard_normal(N).astype(np.float32)
    x2 = rng.standard_normal(N).astype(np.float32)
    y1, _ = oracle.decode_gemv(bits, s0, C, x1, M, N, L, k, V, T)
    y2, _ = oracle.decode_gemv(bits, s0, C, x2, M, N, L, k, V, T)
    y12, _ = oracle.decode_gemv(bits, s0, C, x1.astype(np.float64) + x2, M, N, L, k, V, T)
    assert np.allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12)
    # every decoded weight is a codebook value of its block's path
    assert set(np.unique(What)).issubset(set(C[:, 0].tolist()))

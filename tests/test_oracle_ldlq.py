"""Pins for the error-feedback (LDLQ) oracle, oracle.ldlq_encode.

P1  the page's toy (golden/ldlq_toy.json): targets [0.4, 0.8, 0.2], result [0, 1, 0];
    without feedback (U = I) the result is [0, 0, 0].
P2  diagonal H: U = I, so every block is coded on W itself; the result is bitwise the
    plain weighted encoder with d = diag(H).
P3  proxy-loss identity: for H = U D U^T with U unit upper block-triangular and D
    block diagonal, (w - w_hat) H (w - w_hat)^T equals sum_j eta_j D_j eta_j^T with
    eta_j = t_j - w_hat_j over block j (T = 1: sum_c d_c (t_c - w_hat_c)^2).  A
    transposed U, a wrong sign or feeding back t - w_hat instead of w - w_hat breaks it.
P4  error diffusion: U all ones above the diagonal, a unit-step quantizer and targets
    inside its range keep every running sum of errors within half a step.
P5  causality: a block's code depends only on W's columns up to that block.
P6  feedback lowers the proxy loss against plain rounding on a correlated H, with the
    block factor; the scalar factor with its within-block entries dropped does not (it
    raises the loss many times over), which is why blocks use the block factor.
"""
import json
import os

import numpy as np
import pytest

from trellis_coded_bit_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ldlq_toy.json")


def _spd(rng, N, rho=0.9):
    X = rng.standard_normal((4 * N, N))
    for f in range(1, N):
        X[:, f] = rho * X[:, f - 1] + np.sqrt(1 - rho * rho) * X[:, f]
    return X.T @ X / X.shape[0] + 0.01 * np.eye(N)


def test_toy_from_page(oracle_lib):
    import oracle
    g = json.load(open(GOLDEN))
    page, rd = g["what_the_page_states"], g["reading"]
    H = np.array(rd["H"], float)
    U, d = wl.udu_factor(H)
    assert np.array_equal(U, np.array(rd["U"], float)) and np.array_equal(d, rd["d"])
    W = np.array([page["weights"]], np.float32)
    C = np.array([[0.0], [1.0], [0.0], [1.0]], np.float32)
    _, _, _, what, tgt = oracle.ldlq_encode(W, U, d, C, 2, 1, 1, 1)
    assert np.array_equal(what[0], np.array(page["feedback_result"], np.float32))
    assert np.allclose(tgt[0], page["feedback_targets"], atol=1e-6)
    assert abs(float(W.sum() - what.sum()) - page["feedback_sum_error"]) < 1e-6
    _, _, _, plain, _ = oracle.ldlq_encode(W, np.eye(3), np.ones(3), C, 2, 1, 1, 1)
    assert np.array_equal(plain[0], np.array(page["plain_rounding_to_integers"], np.float32))
    assert abs(float(W.sum() - plain.sum()) - page["plain_rounding_sum_error"]) < 1e-6


@pytest.mark.parametrize("L,k,V,T", [(8, 2, 1, 32), (10, 2, 2, 16)])
def test_diagonal_hessian_is_plain_encoding(oracle_lib, L, k, V, T):
    import oracle
    rng = np.random.default_rng(L + T)
    M, N = 3, 4 * T
    H = np.diag(np.exp(rng.standard_normal(N)))
    U, D = wl.block_udu_factor(H, T)
    d = np.concatenate([np.diag(b) for b in D])
    assert np.array_equal(U, np.eye(N)) and np.allclose(d, np.diag(H), rtol=1e-14, atol=0)
    C = oracle.make_codebook(L, V, 17)
    W = rng.standard_normal((M, N)).astype(np.float32)
    d32 = d.astype(np.float32)
    bits, s0, cost, what, tgt = oracle.ldlq_encode(W, U, d32, C, L, k, V, T)
    pb, ps, pc = oracle.encode_matrix(W, d32, C, L, k, V, T)
    assert np.array_equal(tgt, W)
    assert np.array_equal(bits.reshape(pb.shape), pb)
    assert np.array_equal(s0.reshape(-1), ps)
    assert np.array_equal(cost.reshape(-1).view(np.uint32), pc.view(np.uint32))


@pytest.mark.parametrize("seed,T,L,k,V", [(0, 1, 4, 2, 1), (1, 1, 4, 2, 1), (2, 4, 6, 2, 1),
                                          (3, 8, 8, 2, 2)])
def test_proxy_loss_identity(oracle_lib, seed, T, L, k, V):
    import oracle
    rng = np.random.default_rng(seed)
    N = 24
    H = _spd(rng, N)
    U, D = wl.block_udu_factor(H, T)
    d = np.concatenate([np.diag(b) for b in D])
    U32, d32 = U.astype(np.float32), d.astype(np.float32)
    if T == 1:
        C = (np.arange(16, dtype=np.float32) - 7.5).reshape(16, 1) * np.float32(0.5)
    else:
        C = oracle.make_codebook(L, V, 9)
    W = (2.0 * rng.standard_normal((4, N))).astype(np.float32)
    _, _, _, what, tgt = oracle.ldlq_encode(W, U32, d32, C, L, k, V, T)
    # the identity in exact arithmetic for the fp32 factor actually used
    U64 = U32.astype(np.float64)
    D64 = np.zeros((N, N))
    for j in range(N // T):
        D64[j * T:(j + 1) * T, j * T:(j + 1) * T] = D[j]
    if T == 1:
        D64 = np.diag(d32.astype(np.float64))
    H32 = U64 @ D64 @ U64.T
    for r in range(W.shape[0]):
        e = W[r].astype(np.float64) - what[r]
        eta = tgt[r].astype(np.float64) - what[r]
        lhs = e @ H32 @ e
        rhs = eta @ D64 @ eta
        assert abs(lhs - rhs) <= 1e-4 * max(lhs, 1e-6), (lhs, rhs)


def test_error_diffusion_running_sums(oracle_lib):
    import oracle
    rng = np.random.default_rng(5)
    N = 40
    U = np.triu(np.ones((N, N)))
    C = (np.arange(16, dtype=np.float32) - 8).reshape(16, 1)  # integers -8..7
    W = rng.uniform(-3, 3, size=(3, N)).astype(np.float32)
    _, _, _, what, tgt = oracle.ldlq_encode(W, U, np.ones(N, np.float32), C, 4, 2, 1, 1)
    assert np.all(what == np.round(what))
    run = np.cumsum(W.astype(np.float64) - what, axis=1)
    assert np.max(np.abs(run)) <= 0.5 + 1e-5
    assert np.allclose(tgt[:, 1:] - W[:, 1:], run[:, :-1], atol=1e-5)


def test_causality(oracle_lib):
    import oracle
    rng = np.random.default_rng(8)
    L, k, V, T, N = 8, 2, 1, 16, 64
    U, D = wl.block_udu_factor(_spd(rng, N), T)
    d = np.concatenate([np.diag(b) for b in D])
    C = oracle.make_codebook(L, V, 3)
    W = rng.standard_normal((2, N)).astype(np.float32)
    W2 = W.copy()
    W2[:, 2 * T:] += 1.0
    a = oracle.ldlq_encode(W, U, d, C, L, k, V, T)
    b = oracle.ldlq_encode(W2, U, d, C, L, k, V, T)
    assert np.array_equal(a[0][:, :2], b[0][:, :2]) and np.array_equal(a[1][:, :2], b[1][:, :2])
    assert not np.array_equal(a[0][:, 2:], b[0][:, 2:])


@pytest.mark.parametrize("T", [1, 8])
def test_feedback_lowers_proxy_loss(oracle_lib, T):
    import oracle
    rng = np.random.default_rng(11)
    L, k, V, N, M = 8, 2, 1, 64, 16
    H = _spd(rng, N, rho=0.95)
    U, D = wl.block_udu_factor(H, T)
    d = np.concatenate([np.diag(b) for b in D])
    C = oracle.make_codebook(L, V, 4)
    W = rng.standard_normal((M, N)).astype(np.float32)
    _, _, _, w_fb, _ = oracle.ldlq_encode(W, U, d, C, L, k, V, T)
    _, _, _, w_pl, _ = oracle.ldlq_encode(W, np.eye(N), d, C, L, k, V, T)
    loss = lambda Wh: float(np.einsum("ri,ij,rj->", W - Wh, H, W - Wh))
    assert loss(w_fb) < 0.8 * loss(w_pl)
    if T > 1:
        U1, d1 = wl.udu_factor(H)
        _, _, _, w_sc, _ = oracle.ldlq_encode(W, U1, d1, C, L, k, V, T)
        assert loss(w_sc) > 2.0 * loss(w_pl)

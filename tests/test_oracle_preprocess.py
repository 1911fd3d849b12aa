"""Pins for the pre-processing oracles: oracle.hadamard and oracle.scale_field.

H1  the page's 4x4 example (golden/hadamard_4x4.json): H_4/2 on [3.0, 0.2, -0.1, 0.1]
    gives [1.6, 1.3, 1.6, 1.5], with the sum of squares 9.06 kept.
H2  the matrix equals scipy's Hadamard (Sylvester construction) scaled by 1/sqrt(n).
H3  orthogonality: R R^T = I for random signs; the inverse undoes the forward; norms
    are kept; W x = (W R^T)(R x) (the page's identity).
H4  chunks: a row of several chunks is rotated chunk by chunk.
S1  closed form: for W = sign * alpha_r * beta_c the field recovers alpha_r |beta_c|
    exactly and Wn is the sign pattern; every column of Wn has unit RMS.
S2  equivariance: scaling a row of W scales that row's factor only.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hadamard_4x4.json")


def test_page_example(oracle_lib):
    import oracle
    g = json.load(open(GOLDEN))["what_the_page_states"]
    H = np.array(g["matrix_times_2"], float) * g["scale"]
    x = np.array(g["input"])
    y = oracle.hadamard(x, 4)[0]
    assert np.allclose(y, g["output"], atol=1e-12)
    assert np.allclose(H @ x, y, atol=1e-12)
    assert abs(float(y @ y) - g["sum_of_squares_both"]) < 1e-9
    assert abs(float(x @ x) - g["sum_of_squares_both"]) < 1e-9


@pytest.mark.parametrize("n", [1, 2, 8, 64])
def test_matches_sylvester_construction(oracle_lib, n):
    import oracle
    from scipy.linalg import hadamard
    R = oracle.hadamard(np.eye(n), n)      # row i = R e_i = column i of R
    assert np.allclose(R.T, hadamard(n) / np.sqrt(n), atol=1e-14)


@pytest.mark.parametrize("n", [4, 32, 128])
def test_orthogonal_and_inverse(oracle_lib, n):
    import oracle
    rng = np.random.default_rng(n)
    sigma = rng.choice([-1.0, 1.0], size=n)
    R = oracle.hadamard(np.eye(n), n, sigma).T
    assert np.allclose(R @ R.T, np.eye(n), atol=1e-12)
    X = rng.standard_normal((5, n))
    Y = oracle.hadamard(X, n, sigma)
    assert np.allclose(oracle.hadamard(Y, n, sigma, inverse=True), X, atol=1e-12)
    assert np.allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(X, axis=1), rtol=1e-12)
    # W x = (W R^T)(R x): rows of W and x take the same forward rotation
    W = rng.standard_normal((3, n))
    x = rng.standard_normal(n)
    WRt = oracle.hadamard(W, n, sigma)
    Rx = oracle.hadamard(x, n, sigma)[0]
    assert np.allclose(WRt @ Rx, W @ x, atol=1e-10)


def test_chunks(oracle_lib):
    import oracle
    rng = np.random.default_rng(1)
    sigma = rng.choice([-1.0, 1.0], size=48)
    X = rng.standard_normal((2, 48))
    Y = oracle.hadamard(X, 16, sigma)
    for c in range(3):
        s = slice(16 * c, 16 * c + 16)
        assert np.allclose(Y[:, s], oracle.hadamard(X[:, s], 16, sigma[s]), atol=1e-14)


def test_scale_field_closed_form(oracle_lib):
    import oracle
    rng = np.random.default_rng(2)
    M, N = 7, 12
    alpha = np.exp(rng.standard_normal(M))
    beta = np.exp(rng.standard_normal(N)) * rng.choice([-1, 1], size=N)
    S = rng.choice([-1.0, 1.0], size=(M, N))
    W = (S * alpha[:, None] * beta[None, :]).astype(np.float32)
    a, b, Wn = oracle.scale_field(W)
    W64 = W.astype(np.float64)
    # the float32 W is the exact input; its own field is alpha |beta| up to float32 rounding
    assert np.allclose(np.outer(a, b), np.abs(W64), rtol=2e-7)
    assert np.allclose(np.abs(Wn), 1.0, rtol=2e-7)
    assert np.allclose(np.sqrt((Wn ** 2).mean(axis=0)), 1.0, rtol=1e-12)
    assert np.allclose(a, np.sqrt((W64 ** 2).mean(axis=1)), rtol=1e-12)


def test_scale_field_equivariance(oracle_lib):
    import oracle
    rng = np.random.default_rng(3)
    W = rng.standard_normal((6, 10)).astype(np.float32)
    a, b, Wn = oracle.scale_field(W)
    W2 = W.copy()
    W2[2] *= 4.0          # exact in float32
    a2, b2, Wn2 = oracle.scale_field(W2)
    exp_a = a.copy()
    exp_a[2] *= 4.0
    assert np.allclose(a2, exp_a, rtol=1e-14)
    assert np.allclose(b2, b, rtol=1e-14)
    assert np.allclose(Wn2, Wn, rtol=1e-14, atol=1e-300)
    assert np.allclose(Wn2 * np.outer(a2, b2), W2, rtol=1e-12)

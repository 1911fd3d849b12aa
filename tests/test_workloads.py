"""Seeded input generator: shapes, determinism, and the LDL diagonal."""
import numpy as np

from trellis_coded_bit_amd import workloads as wl


def test_workload_table():
    assert [w.index for w in wl.WORKLOADS] == [0, 1, 2, 3, 4]
    w0, w1, w2, w3, w4 = wl.WORKLOADS
    assert (w0.M, w0.N, w0.L, w0.k, w0.V, w0.T, w0.blocks) == (64, 64, 8, 2, 1, 64, 64)
    assert (w1.M, w1.N, w1.L, w1.k, w1.T, w1.blocks) == (2048, 2048, 16, 2, 256, 16384)
    assert w2.blocks == 65536 and w3.blocks == 229376 and w4.blocks == 229376
    assert (w3.k, w4.k, w4.V) == (3, 2, 2)


def test_weights_deterministic_and_row_ranges():
    w = wl.WORKLOADS[0]
    A = wl.make_weights(w)
    B = wl.make_weights(w)
    assert A.dtype == np.float32 and A.shape == (64, 64)
    assert np.array_equal(A, B)
    part = wl.make_weights(w, rows=slice(10, 20))
    assert np.array_equal(part, A[10:20])
    assert abs(float(A.mean())) < 0.1 and 0.8 < float(A.std()) < 1.2


def test_ldl_diagonal_small():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((300, 40)) * np.exp(rng.standard_normal(40))
    H = wl.hessian_from_samples(X)
    d = wl.ldl_diagonal(H)
    # log det H = sum log d
    sign, logdet = np.linalg.slogdet(H)
    assert sign > 0 and abs(logdet - np.sum(np.log(d))) < 1e-8 * abs(logdet)
    # H = L D L^T with L unit lower triangular, reconstructed explicitly
    R = np.linalg.cholesky(H)
    Lm = R / np.diag(R)[None, :]
    assert np.allclose(np.diag(Lm), 1.0)
    assert np.allclose(Lm @ np.diag(d) @ Lm.T, H, rtol=1e-10, atol=1e-10)
    # d_1 is H_11, and the last pivot is 1 / (H^-1)_nn
    assert abs(d[0] - H[0, 0]) < 1e-12 * H[0, 0]
    assert abs(d[-1] - 1.0 / np.linalg.inv(H)[-1, -1]) < 1e-8 * d[-1]


def test_weighted_workload_d_small_version():
    # the recipe of the weighted workloads at a reduced size: positive, finite, and
    # varying across features
    w = wl.Workload(9, "t", 8, 512, 16, 2, 1, 256, "student_t", nu=4.0, scale_sigma=0.5,
                    weighted=True, ar_rho=0.9, feat_sigma=1.0, n_samples=256)
    d = wl.make_d(w)
    assert d.shape == (512,) and d.dtype == np.float32
    assert np.all(np.isfinite(d)) and np.all(d > 0)
    assert float(d.max() / d.min()) > 10.0
    W = wl.make_weights(w)
    assert W.shape == (8, 512) and np.all(np.isfinite(W))


def test_sample_blocks():
    w = wl.WORKLOADS[1]
    b = wl.sample_blocks(w, 100)
    per_row = w.N // w.T
    assert np.all(np.diff(b) > 0)
    assert set(range(per_row)) <= set(b.tolist())
    assert set(range((w.M - 1) * per_row, w.M * per_row)) <= set(b.tolist())

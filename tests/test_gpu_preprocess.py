"""Pre-processing kernels on the GPU vs. the float64 oracles.

Hadamard (tcq_hadamard): each output is a signed sum of one chunk's n inputs over
log2(n) butterfly levels plus the 1/sqrt(n) and sign multiplies, all in fp32, so
|error| <= (log2(n) + 3) u sum_i |x_i| / sqrt(n) per output (u = 2^-24, sum over the
output's chunk).

Scale field (tcq_scale_field): a_r sums N squares per row (a lane sums N/256 of them,
then 8 tree additions; with 16-byte loads a lane keeps four sums of N/1024 terms and adds
them pairwise, a shorter chain), b_c sums M squares of W/a per column (slabs of M/64 rows,
then 64 slab sums), each followed by a division and a square root; relative bounds
  a: (N/256 + 16) u,   b: (M/64 + 64 + N/256 + 32) u,   Wn: (bound_a + bound_b + 4) u.
"""
import sys

import numpy as np
import pytest

from trellis_coded_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import api  # noqa: E402

U32 = 2.0 ** -24


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _had_tol(X, n):
    rows, length = X.shape
    s = np.abs(X.astype(np.float64)).reshape(rows, length // n, n).sum(axis=2)
    return np.repeat((np.log2(n) + 3) * U32 * s / np.sqrt(n), n, axis=1) + 1e-30


@pytest.mark.parametrize("n,rows,chunks", [(1, 3, 5), (2, 2, 3), (16, 4, 3), (32, 3, 2),
                                           (64, 5, 3), (128, 2, 2), (256, 3, 2),
                                           (1024, 5, 1), (2048, 2, 7), (4096, 9, 2)])
def test_hadamard_parity(oracle_lib, n, rows, chunks):
    import oracle
    _say(f"hadamard n={n} rows={rows} chunks={chunks}")
    rng = np.random.default_rng(n + rows)
    length = n * chunks
    X = rng.standard_normal((rows, length)).astype(np.float32)
    sigma = rng.choice([-1.0, 1.0], size=length).astype(np.float32)
    Xt = torch.from_numpy(X).cuda()
    st = torch.from_numpy(sigma).cuda()
    Y = api.hadamard(Xt, n, st)
    Yi = api.hadamard(Y, n, st, inverse=True)
    torch.cuda.synchronize()
    ref = oracle.hadamard(X, n, sigma.astype(np.float64))
    tol = _had_tol(X, n)
    Yc = Y.cpu().numpy()
    assert np.all(np.abs(Yc - ref) <= tol)
    # the inverse applied to the GPU's output, against the oracle's inverse of that output
    ref_i = oracle.hadamard(Yc, n, sigma.astype(np.float64), inverse=True)
    assert np.all(np.abs(Yi.cpu().numpy() - ref_i) <= _had_tol(Yc, n))
    assert np.allclose(Yi.cpu().numpy(), X, atol=1e-5)


@pytest.mark.parametrize("n", [256, 2048])
def test_hadamard_unaligned_rows(oracle_lib, n):
    """Rows that start 4 bytes past a 16-byte boundary (a column-offset view, odd row
    stride) take the 4-byte-access kernel; aligned rows take the 16-byte one."""
    import oracle
    _say(f"hadamard unaligned n={n}")
    rng = np.random.default_rng(7 * n)
    rows, length = 3, 2 * n
    base = rng.standard_normal((rows, length + 1)).astype(np.float32)
    sigma = rng.choice([-1.0, 1.0], size=length).astype(np.float32)
    Bt = torch.from_numpy(base).cuda()
    Xv = Bt[:, 1:]
    assert Xv.data_ptr() % 16 != 0 and Xv.stride(0) % 4 != 0
    Y = api.hadamard(Xv, n, torch.from_numpy(sigma).cuda())
    torch.cuda.synchronize()
    X = base[:, 1:]
    ref = oracle.hadamard(np.ascontiguousarray(X), n, sigma.astype(np.float64))
    assert np.all(np.abs(Y.cpu().numpy() - ref) <= _had_tol(X, n))


def test_hadamard_page_example_and_in_place(oracle_lib):
    x = torch.tensor([[3.0, 0.2, -0.1, 0.1]], device="cuda")
    api.hadamard(x, 4, out=x)                    # in place, no signs
    torch.cuda.synchronize()
    assert np.allclose(x.cpu().numpy()[0], [1.6, 1.3, 1.6, 1.5], atol=1e-6)


def test_hadamard_full_size_sampled_rows(oracle_lib):
    """4096 x 4096 weights, full-dimension rotation (n = 4096), 12 rows checked."""
    import oracle
    w = wl.WORKLOADS[2]
    W = wl.make_weights(w)
    rng = np.random.default_rng(12)
    sigma = rng.choice([-1.0, 1.0], size=w.N).astype(np.float32)
    Y = api.hadamard(torch.from_numpy(W).cuda(), 4096, torch.from_numpy(sigma).cuda())
    torch.cuda.synchronize()
    Yc = Y.cpu().numpy()
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 10, replace=False)]))
    ref = oracle.hadamard(W[rows], 4096, sigma.astype(np.float64))
    assert np.all(np.abs(Yc[rows] - ref) <= _had_tol(W[rows], 4096))
    # norms are kept
    assert np.allclose(np.linalg.norm(Yc, axis=1), np.linalg.norm(W, axis=1), rtol=1e-4)


def _scale_bounds(M, N):
    """(a, b) relative bounds from the kernels' summation order."""
    return (N / 256 + 16) * U32, (M / 64 + 64 + N / 256 + 32) * U32


def _check_scale(W, a, b, Wn, rows):
    import oracle
    M, N = W.shape
    ra, rb, rWn = oracle.scale_field(W)
    ta, tb = _scale_bounds(M, N)
    _say(f"  a: worst {np.max(np.abs(a - ra) / ra) / ta:.3g} of the bound; "
         f"b: worst {np.max(np.abs(b - rb) / rb) / tb:.3g} of the bound")
    assert np.all(np.abs(a - ra) <= ta * ra)
    assert np.all(np.abs(b - rb) <= tb * rb)
    tw = (ta / U32 + tb / U32 + 4) * U32
    assert np.all(np.abs(Wn[rows] - rWn[rows]) <= tw * np.abs(rWn[rows]) + 1e-37)


@pytest.mark.parametrize("M,N", [(1, 1), (3, 17), (64, 300), (130, 1000), (257, 64),
                                 (33, 1024), (17, 4100), (40, 8192), (9, 14336), (5, 16384)])
def test_scale_field_parity(oracle_lib, M, N):
    _say(f"scale field M={M} N={N}")
    rng = np.random.default_rng(M * 1000 + N)
    W = (rng.standard_t(4, (M, N)) * np.exp(0.5 * rng.standard_normal(M))[:, None]
         * np.exp(0.5 * rng.standard_normal(N))[None, :]).astype(np.float32)
    if M > 2:
        W[1] = 0.0                 # an all-zero row gets scale 1
    a, b, Wn = api.scale_field(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    _check_scale(W, a.cpu().numpy(), b.cpu().numpy(), Wn.cpu().numpy(), np.arange(M))


def test_scale_field_full_size(oracle_lib):
    """The weighted 4096 x 4096 workload carries a row x column scale field."""
    w = wl.WORKLOADS[2]
    W = wl.make_weights(w)
    a, b, Wn = api.scale_field(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, w.M - 1])
    _check_scale(W, a.cpu().numpy(), b.cpu().numpy(), Wn.cpu().numpy(), rows)

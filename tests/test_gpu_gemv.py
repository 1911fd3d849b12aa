"""Fused decode + matrix-vector product (tcq_decode_gemv) vs. the oracle's decode
followed by a float64 product.

Inputs are seeded random bitstreams with start states below 2^(L-kV) (every such
stream is a path of the trellis); nothing comes from the GPU encoder.  Bars (see
gemv_check.py): on exact inputs (codebook on a 1/8 grid, small-integer x) y must equal the
reference bit for bit; on N(0,1) activations and the Gaussian-quantile codebook each row
must lie within gamma_m sum_i |w_i x_i| of it, m the number of roundings a term passes
through in the kernel's summation order.  Each case prints its worst error / bound.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import api  # noqa: E402

import gemv_check as gc  # noqa: E402


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _random_streams(rng, nb, L, k, V, T):
    nw = (k * T + 31) // 32
    bits = rng.integers(0, 1 << 32, size=(nb, nw), dtype=np.uint64).astype(np.uint32)
    tail = k * T % 32
    if tail:
        bits[:, -1] &= np.uint32(((1 << tail) - 1) << (32 - tail))
    s0 = rng.integers(0, 1 << (L - k * V), size=nb, dtype=np.uint64).astype(np.uint32)
    return bits, s0


def _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T, c_shift=0):
    """c_shift > 0 places the codebook c_shift floats into its allocation."""
    bt = torch.from_numpy(bits.view(np.int32)).cuda()
    st = torch.from_numpy(s0.view(np.int32)).cuda()
    flat = torch.from_numpy(np.ascontiguousarray(C).reshape(-1))
    Cbuf = torch.full((flat.numel() + c_shift,), float("nan"), dtype=torch.float32)
    Cbuf[c_shift:] = flat
    Ct = Cbuf.cuda()[c_shift:]
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    y = api.decode_gemv(bt, st, Ct, xt, M, N, L, k, V, T)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(y, yref, What, x, M, N, L, k, V, T):
    m = gc.roundings(M, N, L, k, V, T)
    ratio = gc.bound_ratio(y, yref, What, x, m)
    _say(f"  worst error / bound = {ratio:.3g} (m = {m} roundings)")
    assert ratio <= 1.0, f"error {ratio:.3g} x the bound (m = {m})"


CASES = [
    # L, k, V, T, M, N
    (4, 1, 1, 12, 5, 36),
    (6, 2, 1, 64, 9, 128),
    (8, 2, 2, 32, 8, 96),
    (9, 4, 1, 100, 6, 300),
    (10, 3, 2, 30, 6, 120),
    (12, 4, 2, 64, 3, 128),
    (16, 2, 1, 256, 7, 2048 + 256),
    (16, 3, 1, 256, 5, 1024),
    (16, 2, 2, 256, 4, 768),
    (16, 1, 1, 17, 3, 17 * 61),
    (12, 3, 2, 32, 3, 128),
    (16, 2, 1, 256, 70, 256),
    (12, 2, 1, 64, 4500, 512),   # many short rows: two rows per wave
    (16, 4, 1, 256, 9, 2048),
    # longest blocks (1024 steps)
    (16, 2, 2, 2048, 2, 4096),
    (16, 4, 1, 1024, 2, 2048),
    (16, 2, 1, 1024, 3, 2048),
    (16, 3, 1, 1024, 2, 2048),
]


@pytest.mark.parametrize("L,k,V,T,M,N", CASES)
def test_gemv_parity_small(oracle_lib, L, k, V, T, M, N):
    import oracle
    _say(f"gemv L={L} k={k} V={V} T={T} M={M} N={N}")
    rng = np.random.default_rng(L * 1000 + k * 100 + V * 10 + T)
    C = oracle.make_codebook(L, V, 40 + L)
    bits, s0 = _random_streams(rng, M * (N // T), L, k, V, T)
    x = rng.standard_normal(N).astype(np.float32)
    yref, What = oracle.decode_gemv(bits, s0, C, x, M, N, L, k, V, T)
    y = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    _check(y, yref, What, x, M, N, L, k, V, T)
    # unit vector: exactly the decoded column
    e = np.zeros(N, np.float32)
    e[N - 1] = 1.0
    ye = _gpu_gemv(bits, s0, C, e, M, N, L, k, V, T)
    assert np.array_equal(ye, What[:, N - 1])


@pytest.mark.parametrize("M,N,L,k,V,T", [(2048, 2048, 16, 2, 1, 256),
                                         (14336, 4096, 16, 2, 2, 256),
                                         (4096, 14336, 16, 3, 1, 256)])
def test_gemv_full_size_sampled_rows(oracle_lib, M, N, L, k, V, T):
    """Full-size launch; the oracle checks 64 sampled rows (first, last, random)."""
    import oracle
    _say(f"gemv full M={M} N={N} L={L} k={k} V={V}")
    rng = np.random.default_rng(M + N + k)
    C = oracle.make_codebook(L, V, 3001)
    per_row = N // T
    bits, s0 = _random_streams(rng, M * per_row, L, k, V, T)
    x = rng.standard_normal(N).astype(np.float32)
    y = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
    sel = (rows[:, None] * per_row + np.arange(per_row)[None, :]).reshape(-1)
    yref, What = oracle.decode_gemv(bits[sel], s0[sel], C, x, rows.size, N, L, k, V, T)
    _check(y[rows], yref, What, x, M, N, L, k, V, T)


@pytest.mark.parametrize("L,k,V,T,M,N,c_shift", [(16, 2, 1, 256, 7, 2048 + 256, 1),
                                                   (16, 2, 2, 256, 4, 768, 3),
                                                   (16, 3, 1, 256, 5, 1024, 2)])
def test_gemv_unaligned_codebook(oracle_lib, L, k, V, T, M, N, c_shift):
    """A codebook that does not start on 16 bytes is copied into LDS float by float; the
    result must equal the aligned launch's bit for bit."""
    import oracle
    _say(f"gemv L={L} k={k} V={V} T={T} M={M} N={N} codebook +{c_shift} floats")
    rng = np.random.default_rng(L * 1000 + k * 100 + V * 10 + T + c_shift)
    C = oracle.make_codebook(L, V, 50 + L)
    bits, s0 = _random_streams(rng, M * (N // T), L, k, V, T)
    x = rng.standard_normal(N).astype(np.float32)
    yref, What = oracle.decode_gemv(bits, s0, C, x, M, N, L, k, V, T)
    y = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T, c_shift)
    _check(y, yref, What, x, M, N, L, k, V, T)
    y0 = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))


def test_gemv_empty_and_deterministic(oracle_lib):
    import oracle
    L, k, V, T, M = 16, 2, 1, 256, 3
    C = oracle.make_codebook(L, V, 1)
    Ct = torch.from_numpy(C).cuda()
    empty_i = torch.empty(0, dtype=torch.int32, device="cuda")
    y = api.decode_gemv(empty_i, empty_i, Ct, torch.empty(0, device="cuda"), M, 0, L, k, V, T)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), np.zeros(M, np.float32))
    rng = np.random.default_rng(9)
    N = 4096
    bits, s0 = _random_streams(rng, M * N // T, L, k, V, T)
    x = rng.standard_normal(N).astype(np.float32)
    y1 = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    y2 = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


EXACT_CASES = [
    # M, N, L, k, V, T
    (2048, 2048, 16, 2, 1, 256),
    (14336, 4096, 16, 2, 2, 256),
    (4096, 14336, 16, 3, 1, 256),
    (9, 2048, 16, 4, 1, 256),
    (3, 17 * 61, 16, 1, 1, 17),     # generic kernel
    (5, 960, 12, 3, 2, 120),        # generic kernel (blocks not whole units)
    (4500, 512, 12, 2, 1, 64),
]


@pytest.mark.parametrize("M,N,L,k,V,T", EXACT_CASES)
def test_gemv_exact_arithmetic(oracle_lib, M, N, L, k, V, T):
    """Every product and partial sum is an fp32 number, so any summation order gives the
    exact sum: every row must equal the reference bit for bit.  A dropped, doubled or
    misplaced term shows up as a mismatch."""
    import oracle
    if N % T:
        pytest.skip("shape")
    _say(f"gemv exact M={M} N={N} L={L} k={k} V={V} T={T} "
         f"({'column' if gc.col_plan(M, N, L, k, V, T) else 'generic'} kernel)")
    rng = np.random.default_rng(M * 7 + N + k * 3 + V)
    C = gc.grid_codebook(oracle.make_codebook(L, V, 3001))
    bits, s0 = _random_streams(rng, M * (N // T), L, k, V, T)
    x = rng.integers(-8, 9, N).astype(np.float32)
    y = _gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    yref, _ = oracle.decode_gemv(bits, s0, C, x, M, N, L, k, V, T)
    bad = np.nonzero(y.astype(np.float64) != yref)[0]
    assert gc.exact_equal(y, yref), (f"{bad.size} rows differ; first row {bad[0]}: gpu "
                                     f"{y[bad[0]]!r} ref {yref[bad[0]]!r}")

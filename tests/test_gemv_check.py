"""The decode-GEMV comparisons themselves (CPU only): they accept a correct fp32 sum in any
order and reject a sum with one term dropped."""
import numpy as np
import pytest

import gemv_check as gc


def _problem(rng, L, k, V, T, M, N, exact):
    import oracle
    C = oracle.make_codebook(L, V, 11)
    if exact:
        C = gc.grid_codebook(C)
        x = rng.integers(-8, 9, N).astype(np.float32)
    else:
        x = rng.standard_normal(N).astype(np.float32)
    nb = M * (N // T)
    nw = (k * T + 31) // 32
    bits = rng.integers(0, 1 << 32, size=(nb, nw), dtype=np.uint64).astype(np.uint32)
    s0 = rng.integers(0, 1 << (L - k * V), size=nb, dtype=np.uint64).astype(np.uint32)
    yref, What = oracle.decode_gemv(bits, s0, C, x, M, N, L, k, V, T)
    return yref, What, x


def _fp32_sum_in_order(What, x, order):
    """y[r] = sum of fl(w x) terms in the given order, fp32 throughout (fmaf chain)."""
    M, N = What.shape
    y = np.zeros(M, np.float32)
    for r in range(M):
        acc = np.float32(0)
        for i in order:
            acc = np.float32(np.float64(What[r, i]) * np.float64(x[i]) + np.float64(acc))
        y[r] = acc
    return y


@pytest.mark.parametrize("exact", [False, True])
def test_checks_accept_fp32_sums_and_reject_a_dropped_term(exact):
    rng = np.random.default_rng(5 + exact)
    L, k, V, T, M, N = 8, 2, 1, 64, 6, 512
    yref, What, x = _problem(rng, L, k, V, T, M, N, exact)
    m = gc.roundings(M, N, L, k, V, T)
    # two different fp32 orders, each within the bound (and exact on the exact inputs)
    for order in (np.arange(N), rng.permutation(N)):
        y = _fp32_sum_in_order(What, x, order)
        assert gc.bound_ratio(y, yref, What, x, N) <= 1.0
        if exact:
            assert gc.exact_equal(y, yref)
    # the kernel's bound m is much tighter than N roundings
    assert m < N // 8
    # plant a drop: row 2 loses its largest term
    r = 2
    i = int(np.argmax(np.abs(What[r].astype(np.float64) * x)))
    bad = yref.copy()
    bad[r] -= np.float64(What[r, i]) * np.float64(x[i])
    bad32 = bad.astype(np.float32)
    assert gc.bound_ratio(bad32, yref, What, x, m) > 1.0
    if exact:
        assert not gc.exact_equal(bad32, yref)
    # a dropped small term is caught by the exact comparison
    if exact:
        j = int(np.nonzero(np.abs(What[r] * x) == 0.125)[0][0]) if np.any(
            np.abs(What[r] * x) == 0.125) else i
        bad = yref.copy()
        bad[r] -= np.float64(What[r, j]) * np.float64(x[j])
        assert not gc.exact_equal(bad.astype(np.float32), yref)


def test_plan_of_the_benchmark_shapes():
    # 2048 x 2048, k = 2: 128 one-word units per row, one unit per thread, 2 waves per row
    assert gc.col_plan(2048, 2048, 16, 2, 1, 256) == (1, 16, 128)
    # rows of more than 1024 units take the generic kernel
    assert gc.col_plan(4, 32768, 16, 2, 1, 256) is None
    assert gc.roundings(2048, 2048, 16, 2, 1, 256) == 16 + 6 + 1
    # 14336 x 4096, k = 2, V = 2: 256 units per row, 4 waves per row
    assert gc.col_plan(14336, 4096, 16, 2, 2, 256) == (1, 8, 256)
    assert gc.roundings(14336, 4096, 16, 2, 2, 256) == 16 + 6 + 3
    # 4096 x 14336, k = 3: 448 units of 3 words (32 steps), 7 waves per row
    assert gc.col_plan(4096, 14336, 16, 3, 1, 256) == (1, 32, 448)
    assert gc.roundings(4096, 14336, 16, 3, 1, 256) == 32 + 6 + 6
    # blocks that are not whole units take the generic kernel
    assert gc.col_plan(3, 17 * 61, 16, 1, 1, 17) is None


def test_exact_inputs_are_exact_in_fp32():
    # the largest exact case: 14336 columns, |c| <= 4 on a 1/8 grid, |x| <= 8 -- every
    # partial sum is a multiple of 1/8 below 2^19 in magnitude, i.e. an fp32 number
    assert 14336 * 4 * 8 * 8 < 2 ** 24

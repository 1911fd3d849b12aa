"""A seeded random sweep over the whole supported shape space, against the oracle:
2 <= L <= 16, k*V < L, k*V <= 8, V in {1, 2, 4}, strided rows, Gaussian / heavy-tailed /
dyadic (tie-rich) weights, weighted and unweighted, quantile and random codebooks.
Per case: encode with reconstruction (parity rule of tests/parity.py, reconstruction
bitwise equal to the oracle's decode), decode-GEMV (error bound of gemv_check.py) and,
where the float64 oracle is quick (L <= 12, k*V <= 4), the soft trellis (bounds of
test_gpu_bcjr.py)."""
import sys

import numpy as np
import pytest

import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import api  # noqa: E402

import test_gpu_bcjr as tb  # noqa: E402
import test_gpu_gemv as tg  # noqa: E402

CASES = 80


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _draw(rng):
    """One random case; None when the drawn (L, V) admits no k."""
    L = int(rng.choice([16, 16, 16] + list(range(2, 16))))
    V = int(rng.choice([1, 1, 1, 2, 2, 4]))
    while V > L - 1:
        V = max(1, V // 2)
    kmax = min(8 // V, (L - 1) // V)
    if kmax < 1:
        return None
    k = int(rng.integers(1, kmax + 1))
    n = int(rng.integers(1, (48 if L >= 15 else 64 if L >= 12 else 300) + 1))
    T = n * V
    M = int(rng.integers(1, 5))
    bpr = int(rng.integers(1, 4))
    N = T * bpr
    pad = int(rng.integers(0, 4))
    weighted = bool(rng.integers(0, 2))
    kind = int(rng.integers(0, 3))
    if kind == 0:
        W = rng.standard_normal((M, N + pad))
    elif kind == 1:
        W = rng.standard_t(3, (M, N + pad)) * 2.0
    else:  # dyadic values: exact arithmetic, many ties
        W = rng.integers(-8, 9, (M, N + pad)) / 4.0
    W = W.astype(np.float32)
    if not weighted:
        d = None
    elif kind == 2:
        d = (2.0 ** rng.integers(-2, 3, N)).astype(np.float32)
    else:
        d = np.exp(0.5 * rng.standard_normal(N)).astype(np.float32)
    return L, k, V, T, M, N, pad, W, d, kind


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(oracle_lib, case):
    import oracle
    rng = np.random.default_rng(7000 + case)
    drawn = _draw(rng)
    while drawn is None:
        drawn = _draw(rng)
    L, k, V, T, M, N, pad, W, d, kind = drawn
    if rng.integers(0, 2):
        C = oracle.make_codebook(L, V, int(rng.integers(1, 10 ** 6)))
    elif kind == 2:
        C = (rng.integers(-4, 5, (1 << L) * V) / 2.0).astype(np.float32)
    else:
        C = rng.standard_normal((1 << L) * V).astype(np.float32)
    C = np.ascontiguousarray(C, dtype=np.float32).reshape(-1)
    _say(f"sweep case {case}: L={L} k={k} V={V} T={T} M={M} N={N} pad={pad} "
         f"weighted={d is not None} kind={kind}")
    Wt = torch.from_numpy(W).cuda()[:, :N]             # rows of stride N + pad
    out = api.encode(Wt, None if d is None else torch.from_numpy(d).cuda(),
                     torch.from_numpy(C).cuda(), L, k, V, T, recon=True)
    torch.cuda.synchronize()
    Wn = np.ascontiguousarray(W[:, :N])
    nb = M * (N // T)
    rep = parity.compare(oracle, Wn, d, C, L, k, V, T, np.arange(nb),
                         out.bitstream.cpu().numpy(), out.start_state.cpu().numpy(),
                         out.cost.cpu().numpy(), threads=8)
    assert not rep.failures, rep.failures[:3]
    bits = out.bitstream.cpu().numpy().view(np.uint32).reshape(nb, -1)
    s0 = out.start_state.cpu().numpy().view(np.uint32)
    ref = oracle.decode_matrix(bits, s0, C, M, N, L, k, V, T).astype(np.float32)
    assert np.array_equal(out.recon.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    x = rng.standard_normal(N).astype(np.float32)
    y = tg._gpu_gemv(bits, s0, C, x, M, N, L, k, V, T)
    yref, What = oracle.decode_gemv(bits, s0, C, x, M, N, L, k, V, T)
    tg._check(y, yref, What, x, M, N, L, k, V, T)
    if k * V <= 4 and L <= 12 and kind != 2:
        tau = float(rng.choice([0.05, 0.3, 2.0]))
        soft, logz = tb._gpu(Wn, d, C, L, k, V, T, tau)
        tb._check(soft, logz, Wn, d, C, L, k, V, T, tau, np.arange(nb))

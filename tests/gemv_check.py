"""Comparison of tcq_decode_gemv's y = W_hat x with the oracle's reference (decode of
every block, then a float64 matrix-vector product).

Two bars:

- exact: on inputs where every product and every partial sum is an fp32 number (codebook
  on a 1/8 grid with |c| <= 4, x small integers), any summation order gives the exact
  sum, so y must equal the reference bit for bit;
- bound: on general inputs, every term w_i x_i of a row reaches y[r] through at most m
  roundings (its own fmaf and the additions after it on the way to y[r]), so
  |y[r] - ref[r]| <= gamma_m * sum_i |w_i x_i| with gamma_m = m u / (1 - m u),
  u = 2^-24 (the standard bound for a sum in any fixed order).

m follows the order the kernels sum in, which is fixed by the launch plan of
tcq_decode_gemv for the shape (restated here; see the kernel file):

- column kernel (every block a whole number of units of U = kV / gcd(kV, 32) words, at
  most 1024 units per row, one unit per thread: G = 1): a thread's chain holds at most
  G S V nonzero terms (S = 32 U / kV steps of V coordinates; steps outside the codebook
  part of a pass add an exact 0), then a 6-level shuffle tree over the wave, then the
  row's NT / 64 wave sums added in order: m = G S V + 6 + NT / 64 - 1;
- generic kernel: per pass a lane's chain over its words (at most ceil(words per row / 64),
  each with at most 32 // kV + 1 steps of V coordinates), the 6-level shuffle tree, and the
  P pass sums added to y[r] in order: m = chain + 6 + P - 1.
"""
from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -24
COL_THREADS = 1024
COL_KV = (1, 2, 3, 4, 6, 8)
PART_BYTES = 128 << 10


def col_plan(M, N, L, k, V, T):
    """(G, S, NT) of the column kernel for this shape, or None for the generic kernel."""
    kv = k * V
    n = T // V
    nwords = (k * T + 31) // 32
    wpr = (N // T) * nwords
    Uw = kv // math.gcd(kv, 32)
    S = 32 * Uw // kv
    whole = wpr > 0 and nwords % Uw == 0 and kv * n == nwords * 32
    if not whole or kv not in COL_KV or V not in (1, 2, 4):
        return None
    upr = wpr // Uw
    nt = COL_THREADS if upr >= COL_THREADS else (upr + 63) // 64 * 64
    G = -(-upr // nt)
    if G > 1:
        return None
    return G, S, nt


def roundings(M, N, L, k, V, T):
    """Largest number of roundings a term passes through on its way to y[r]."""
    plan = col_plan(M, N, L, k, V, T)
    if plan is not None:
        G, S, nt = plan
        return G * S * V + 6 + nt // 64 - 1
    kv = k * V
    nwords = (k * T + 31) // 32
    wpr = (N // T) * nwords
    plog = 0
    while plog < L and (2 << plog) * V * 4 <= PART_BYTES:
        plog += 1
    parts = 1 << (L - plog)
    chain = -(-wpr // 64) * (32 // kv + 1) * V
    return chain + 6 + parts - 1


def bound(What, x, m):
    """gamma_m * sum_i |w_i x_i| per row (float64)."""
    g = m * U / (1.0 - m * U)
    return g * (np.abs(What.astype(np.float64)) @ np.abs(np.asarray(x, dtype=np.float64)))


def bound_ratio(y, yref, What, x, m):
    """max over rows of |y - ref| / bound (<= 1 passes)."""
    err = np.abs(np.asarray(y, dtype=np.float64) - yref)
    b = bound(What, x, m) + 1e-300
    return float(np.max(err / b)) if err.size else 0.0


def exact_equal(y, yref):
    """y equals the exactly representable reference bit for bit."""
    ref32 = np.asarray(yref, dtype=np.float64).astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), yref), "reference is not an fp32 number"
    return np.array_equal(np.asarray(y, dtype=np.float32), ref32)


def grid_codebook(C):
    """A codebook on the 1/8 grid with |c| <= 4 (the given table rounded and clipped)."""
    return np.clip(np.round(np.asarray(C, dtype=np.float64) * 8) / 8, -4, 4).astype(np.float32)

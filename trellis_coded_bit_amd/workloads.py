"""Seeded synthetic workloads for the trellis encoder (inputs only).

This module produces encoder *inputs*: weight matrices W and per-column weights d.
It contains none of the encoder's arithmetic; both the GPU path and the CPU oracle
consume what it returns.  The codebook is not made here (it is part of the method:
``tcq_make_codebook`` in the library, ``make_codebook`` in the oracle).

The matrices stand in for the real projection weights the pages quantize (1B- to
8B-class layers); no dataset or checkpoint is involved.  d is the diagonal of the LDL
factorization of a layer Hessian H = X^T X / n built from synthetic inputs X (the
CurveTQ abstract names the LDL diagonal as the per-coordinate weight; the Pingala-8
post defines H as the average of x x^T over inputs).

Generation is numpy PCG64 (`default_rng(seed)`) in float64, cast to float32 at the end.
Seeds: W uses 1000+i, d uses 2000+i, the codebook uses 3000+i (i = workload index).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    N: int
    L: int
    k: int
    V: int
    T: int
    w_kind: str          # "normal" or "student_t"
    nu: float = 0.0      # Student-t degrees of freedom
    scale_sigma: float = 0.0  # factored row x column log-normal scale field (0: none)
    weighted: bool = False    # d from a synthetic Hessian (False: d == 1)
    ar_rho: float = 0.0
    feat_sigma: float = 0.0
    n_samples: int = 2048

    @property
    def blocks(self) -> int:
        return self.M * (self.N // self.T)

    @property
    def weights(self) -> int:
        return self.M * self.N

    @property
    def w_seed(self) -> int:
        return 1000 + self.index

    @property
    def d_seed(self) -> int:
        return 2000 + self.index

    @property
    def codebook_seed(self) -> int:
        return 3000 + self.index


WORKLOADS = [
    Workload(0, "tiny-L8-64x64", 64, 64, 8, 2, 1, 64, "normal"),
    Workload(1, "llama3.2-1b-proj-2048x2048-L16k2", 2048, 2048, 16, 2, 1, 256, "normal"),
    Workload(2, "weighted-4096x4096-L16k2", 4096, 4096, 16, 2, 1, 256, "student_t", nu=4.0,
             scale_sigma=0.5, weighted=True, ar_rho=0.9, feat_sigma=1.0),
    Workload(3, "k3-4096x14336-L16k3", 4096, 14336, 16, 3, 1, 256, "student_t", nu=4.0,
             scale_sigma=0.5, weighted=True, ar_rho=0.9, feat_sigma=1.0),
    Workload(4, "8b-mlp-14336x4096-L16k2V2", 14336, 4096, 16, 2, 2, 256, "student_t", nu=5.0,
             weighted=True, ar_rho=0.8, feat_sigma=1.0),
]


def make_weights(wl: Workload, rows: slice | None = None) -> np.ndarray:
    """W (float32, M x N row-major).  `rows` restricts to a row range; the values of
    every row do not depend on which rows are requested."""
    rng = np.random.default_rng(wl.w_seed)
    M, N = wl.M, wl.N
    if wl.scale_sigma > 0:
        zr = rng.standard_normal(M)
        zc = rng.standard_normal(N)
        row_scale = np.exp(wl.scale_sigma * zr)
        col_scale = np.exp(wl.scale_sigma * zc)
    r0, r1 = (0, M) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else M)
    out = np.empty((r1 - r0, N), dtype=np.float32)
    # rows are drawn from per-row child generators so any row range is reproducible
    ss = np.random.SeedSequence(wl.w_seed).spawn(M)
    for i, r in enumerate(range(r0, r1)):
        g = np.random.default_rng(ss[r])
        if wl.w_kind == "normal":
            row = g.standard_normal(N)
        else:
            row = g.standard_t(wl.nu, N)
        if wl.scale_sigma > 0:
            row = row * row_scale[r] * col_scale
        out[i] = row.astype(np.float32)
    return out


def hessian_from_samples(X: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """H = X^T X / n, damped by damp * mean(diag H) on the diagonal (float64)."""
    n = X.shape[0]
    H = X.T @ X / n
    lam = damp * float(np.mean(np.diag(H)))
    H[np.diag_indices_from(H)] += lam
    return H


def ldl_diagonal(H: np.ndarray) -> np.ndarray:
    """diag(D) of H = L D L^T with L unit lower-triangular, natural order (float64).
    Via Cholesky H = R R^T: L = R diag(R)^-1 and D = diag(R)^2."""
    R = np.linalg.cholesky(H)
    return np.diag(R) ** 2


def udu_factor(H: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """H = U diag(d) U^T with U unit upper-triangular (float64), the factor that error
    feedback in natural column order uses.  It is the LDL factorization of H in reversed
    feature order: with P the reversal, P H P = R R^T (Cholesky), U = P R P diag(R)^-1
    reversed, d = diag(R)^2 reversed."""
    R = np.linalg.cholesky(H[::-1, ::-1])
    r = np.diag(R).copy()
    U = (R / r[None, :])[::-1, ::-1].copy()
    return U, (r ** 2)[::-1].copy()


def block_udu_factor(H: np.ndarray, T: int) -> tuple[np.ndarray, np.ndarray]:
    """H = U D U^T with U unit upper block-triangular (identity T x T diagonal blocks)
    and D block diagonal (float64): the factor error feedback over coding blocks of T
    columns uses.  From the scalar factor H = U1 diag(d1) U1^T: the diagonal blocks
    B_j of U1 give D_j = B_j diag(d1_j) B_j^T and U = U1 blockdiag(B)^-1.
    Returns (U, D) with D as an array of the N/T diagonal blocks, shape (N/T, T, T).
    T = 1 gives the scalar factor."""
    N = H.shape[0]
    assert N % T == 0
    U1, d1 = udu_factor(H)
    U = np.empty_like(U1)
    D = np.empty((N // T, T, T))
    for j in range(N // T):
        s = slice(j * T, (j + 1) * T)
        B = U1[s, s]
        D[j] = (B * d1[s][None, :]) @ B.T
        Binv = np.linalg.inv(B)
        U[:j * T + T, s] = U1[:j * T + T, s] @ Binv
        U[j * T + T:, s] = 0.0
        U[s, s] = np.eye(T)
    return U, D


def make_ldlq_inputs(wl: Workload, N: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(U, d) as float32 for error feedback over the workload's synthetic Hessian, with
    U the block factor of block_udu_factor and d the diagonal of its D.  `N` restricts
    to the first N features (for smaller tests)."""
    X = make_samples(wl)
    if N is not None:
        X = X[:, :N]
    H = hessian_from_samples(X)
    del X
    U, D = block_udu_factor(H, wl.T)
    d = np.concatenate([np.diag(b) for b in D])
    return U.astype(np.float32), d.astype(np.float32)


def make_samples(wl: Workload) -> np.ndarray:
    """X: n_samples x N, rows AR(1) across the feature index with coefficient rho,
    then feature f scaled by exp(feat_sigma * u_f), u_f ~ N(0, 1)."""
    rng = np.random.default_rng(wl.d_seed)
    n, F, rho = wl.n_samples, wl.N, wl.ar_rho
    X = np.empty((n, F), dtype=np.float64)
    eps = rng.standard_normal((n, F))
    X[:, 0] = eps[:, 0]
    a = np.sqrt(1.0 - rho * rho)
    for f in range(1, F):
        X[:, f] = rho * X[:, f - 1] + a * eps[:, f]
    u = rng.standard_normal(F)
    X *= np.exp(wl.feat_sigma * u)[None, :]
    return X


def make_d(wl: Workload) -> np.ndarray | None:
    """Per-column weights (float32, length N), or None for d == 1."""
    if not wl.weighted:
        return None
    X = make_samples(wl)
    H = hessian_from_samples(X)
    del X
    d = ldl_diagonal(H)
    return d.astype(np.float32)


def sample_blocks(wl: Workload, count: int, seed: int = 7) -> np.ndarray:
    """Seeded uniform sample of block indices plus every block of rows 0 and M-1."""
    per_row = wl.N // wl.T
    rng = np.random.default_rng(seed)
    pick = rng.choice(wl.blocks, size=min(count, wl.blocks), replace=False)
    edge = np.concatenate([np.arange(per_row), (wl.M - 1) * per_row + np.arange(per_row)])
    return np.unique(np.concatenate([pick, edge])).astype(np.int64)


def random_small(seed: int, M: int, N: int, weighted: bool, scale: float = 1.0):
    """Small random problem (W, d) for parity sweeps."""
    rng = np.random.default_rng(seed)
    W = (scale * rng.standard_normal((M, N))).astype(np.float32)
    d = None
    if weighted:
        d = np.exp(rng.standard_normal(N)).astype(np.float32)
    return W, d

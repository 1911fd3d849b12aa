"""ctypes front end of the C oracle (tcq_oracle.c).

TEST INFRASTRUCTURE ONLY.  Argument marshalling lives here; every number is computed
by the C code, which follows the pages' definitions step by step (see the header of
tcq_oracle.c for the passages and the fp32 evaluation order).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tcq_oracle.c")
_LIB = os.path.join(_HERE, "libtcq_oracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f64p = ctypes.POINTER(ctypes.c_double)
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    lib.oracle_inv_normal_cdf.restype = ctypes.c_double
    lib.oracle_inv_normal_cdf.argtypes = [ctypes.c_double]
    lib.oracle_splitmix64_next.restype = ctypes.c_uint64
    lib.oracle_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.oracle_make_codebook.restype = ctypes.c_int
    lib.oracle_make_codebook.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64, _f32p]
    lib.oracle_encode_block.restype = ctypes.c_int
    lib.oracle_encode_block.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, _u32p,
                                        _u32p, _f32p]
    lib.oracle_two_best_block.restype = ctypes.c_int
    lib.oracle_two_best_block.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p,
                                          _f32p]
    lib.oracle_decode_block.restype = None
    lib.oracle_decode_block.argtypes = [_u32p, ctypes.c_uint32, _f32p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
    lib.oracle_path_cost.restype = ctypes.c_float
    lib.oracle_path_cost.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, _u32p, ctypes.c_uint32]
    lib.oracle_ldlq_row.restype = ctypes.c_int
    lib.oracle_ldlq_row.argtypes = [_f32p, _f32p, ctypes.c_long, _f32p, _f32p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                    _u32p, _u32p, _f32p, _f32p, _f32p]
    lib.oracle_bcjr_block.restype = ctypes.c_int
    lib.oracle_bcjr_block.argtypes = [_f64p, _f64p, _f32p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_double, _f64p,
                                      _f64p]
    lib.oracle_hadamard_row.restype = ctypes.c_int
    lib.oracle_hadamard_row.argtypes = [_f64p, ctypes.c_long, ctypes.c_long, _f64p,
                                        ctypes.c_int, _f64p]
    lib.oracle_scale_field.restype = ctypes.c_int
    lib.oracle_scale_field.argtypes = [_f32p, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                       _f64p, _f64p, _f64p]
    _lib = lib
    return lib


def _fp(a):
    return None if a is None else a.ctypes.data_as(_f32p)


def _up(a):
    return a.ctypes.data_as(_u32p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def nwords(k: int, T: int) -> int:
    return (k * T + 31) // 32


def inv_normal_cdf(p: float) -> float:
    return _load().oracle_inv_normal_cdf(float(p))


def splitmix64_stream(seed: int, count: int) -> list[int]:
    st = ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF)
    lib = _load()
    return [lib.oracle_splitmix64_next(ctypes.byref(st)) for _ in range(count)]


def make_codebook(L: int, V: int, seed: int) -> np.ndarray:
    out = np.empty((1 << L, V), dtype=np.float32)
    rc = _load().oracle_make_codebook(L, V, seed, _fp(out))
    if rc != 0:
        raise ValueError(f"oracle_make_codebook failed ({rc})")
    return out


def encode_block(w, d, C, L, k, V, T, fixed_s0=-1):
    """Returns (bits uint32[nwords], s0, cost)."""
    w = _f32(w)
    d = _f32(d)
    C = _f32(C)
    assert w.size == T and (d is None or d.size == T) and C.size == (1 << L) * V
    bits = np.zeros(nwords(k, T), dtype=np.uint32)
    s0 = ctypes.c_uint32(0)
    cost = ctypes.c_float(0)
    rc = _load().oracle_encode_block(_fp(w), _fp(d), _fp(C), L, k, V, T, fixed_s0,
                                     _up(bits), ctypes.byref(s0), ctypes.byref(cost))
    if rc != 0:
        raise ValueError(f"oracle_encode_block failed ({rc})")
    return bits, int(s0.value), np.float32(cost.value)


def two_best_block(w, d, C, L, k, V, T, fixed_s0=-1):
    w = _f32(w)
    d = _f32(d)
    C = _f32(C)
    best = ctypes.c_float(0)
    second = ctypes.c_float(0)
    rc = _load().oracle_two_best_block(_fp(w), _fp(d), _fp(C), L, k, V, T, fixed_s0,
                                       ctypes.byref(best), ctypes.byref(second))
    if rc != 0:
        raise ValueError(f"oracle_two_best_block failed ({rc})")
    return np.float32(best.value), np.float32(second.value)


def decode_block(bits, s0, C, L, k, V, T):
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    C = _f32(C)
    out = np.empty(T, dtype=np.float32)
    _load().oracle_decode_block(_up(bits), s0, _fp(C), L, k, V, T, _fp(out))
    return out


def path_cost(w, d, C, L, k, V, T, bits, s0):
    w = _f32(w)
    d = _f32(d)
    C = _f32(C)
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    return np.float32(_load().oracle_path_cost(_fp(w), _fp(d), _fp(C), L, k, V, T,
                                                _up(bits), s0))


def encode_matrix(W, d, C, L, k, V, T, blocks=None, threads=1):
    """Encode coding blocks of a row-major M x N matrix.

    Block b = r * (N // T) + c covers W[r, c*T:(c+1)*T] and d[c*T:(c+1)*T].
    `blocks` selects a subset (default: all).  Blocks are independent; `threads` > 1
    runs whole blocks on a thread pool (each block is still single-threaded).
    Returns (bits [nb, nwords], s0 [nb], cost [nb]) for the selected blocks.
    """
    W = np.asarray(W, dtype=np.float32)
    M, N = W.shape
    assert N % T == 0
    per_row = N // T
    if blocks is None:
        blocks = np.arange(M * per_row)
    blocks = np.asarray(blocks, dtype=np.int64)
    nb = blocks.size
    bits = np.zeros((nb, nwords(k, T)), dtype=np.uint32)
    s0 = np.zeros(nb, dtype=np.uint32)
    cost = np.zeros(nb, dtype=np.float32)
    C = _f32(C)
    dd = _f32(d)

    def one(i):
        b = int(blocks[i])
        r, c = divmod(b, per_row)
        wb = np.ascontiguousarray(W[r, c * T:(c + 1) * T])
        db = None if dd is None else np.ascontiguousarray(dd[c * T:(c + 1) * T])
        bb, ss, cc = encode_block(wb, db, C, L, k, V, T)
        bits[i] = bb
        s0[i] = ss
        cost[i] = cc

    if threads <= 1:
        for i in range(nb):
            one(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(nb)))
    return bits, s0, cost


def decode_matrix(bits, s0, C, M, N, L, k, V, T):
    """Reconstruction of an M x N matrix from per-block bitstreams (oracle decode of
    every block, placed at W[r, c*T:(c+1)*T] for block r*(N/T)+c)."""
    per_row = N // T
    out = np.empty((M, N), dtype=np.float32)
    bits = np.asarray(bits).view(np.uint32).reshape(M * per_row, -1)
    s0 = np.asarray(s0).view(np.uint32).reshape(-1)
    for b in range(M * per_row):
        r, c = divmod(b, per_row)
        out[r, c * T:(c + 1) * T] = decode_block(bits[b], int(s0[b]), C, L, k, V, T)
    return out


def decode_gemv(bits, s0, C, x, M, N, L, k, V, T):
    """y = W_hat x for the decoded matrix W_hat, accumulated in float64 (the plain
    definition: decode every block, then a matrix-vector product)."""
    What = decode_matrix(bits, s0, C, M, N, L, k, V, T)
    return What.astype(np.float64) @ np.asarray(x, dtype=np.float64), What


def ldlq_encode(W, U, d, C, L, k, V, T, rows=None, threads=1):
    """Error-feedback (LDLQ) encoding of the selected rows of W (default: all).

    U is N x N float32, unit upper triangular with H = U diag(d) U^T; only entries
    U[i, c] whose column block is later than the row's block are used.  Returns
    (bits [rows, N/T, nwords], s0 [rows, N/T], cost [rows, N/T], W_hat [rows, N],
    targets [rows, N]) as computed by tcq_oracle.c's oracle_ldlq_row.
    """
    W = np.asarray(W, dtype=np.float32)
    M, N = W.shape
    assert N % T == 0
    U = np.ascontiguousarray(U, dtype=np.float32)
    assert U.shape == (N, N)
    dd = _f32(d)
    C = _f32(C)
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    nblk = N // T
    R = rows.size
    bits = np.zeros((R, nblk, nwords(k, T)), dtype=np.uint32)
    s0 = np.zeros((R, nblk), dtype=np.uint32)
    cost = np.zeros((R, nblk), dtype=np.float32)
    what = np.zeros((R, N), dtype=np.float32)
    tgt = np.zeros((R, N), dtype=np.float32)
    lib = _load()

    def one(i):
        w = np.ascontiguousarray(W[int(rows[i])])
        rc = lib.oracle_ldlq_row(_fp(w), _fp(U), N, _fp(dd), _fp(C), L, k, V, T, N,
                                 _up(bits[i]), _up(s0[i]), _fp(cost[i]), _fp(what[i]),
                                 _fp(tgt[i]))
        if rc != 0:
            raise ValueError(f"oracle_ldlq_row failed ({rc})")

    if threads <= 1:
        for i in range(R):
            one(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(R)))
    return bits, s0, cost, what, tgt


def bcjr_block(w, d, C, L, k, V, T, tau):
    """Soft codeword (float64 [T]) and log Z (natural log) of one block at temperature
    tau; w and d are taken in float64 (pass float32 data to match the GPU's inputs)."""
    f64p = ctypes.POINTER(ctypes.c_double)
    w = np.ascontiguousarray(w, dtype=np.float64)
    dd = None if d is None else np.ascontiguousarray(d, dtype=np.float64)
    C = _f32(C)
    assert w.size == T and C.size == (1 << L) * V
    soft = np.empty(T, dtype=np.float64)
    logz = ctypes.c_double(0)
    rc = _load().oracle_bcjr_block(w.ctypes.data_as(f64p),
                                   None if dd is None else dd.ctypes.data_as(f64p), _fp(C),
                                   L, k, V, T, float(tau), soft.ctypes.data_as(f64p),
                                   ctypes.byref(logz))
    if rc != 0:
        raise ValueError(f"oracle_bcjr_block failed ({rc})")
    return soft, float(logz.value)


def bcjr_matrix(W, d, C, L, k, V, T, tau, blocks=None, threads=1):
    """Soft codewords [nb, T] and log Z [nb] for the selected blocks of W (block
    b = r*(N/T)+c covers W[r, cT:(c+1)T] and d[cT:(c+1)T])."""
    W = np.asarray(W, dtype=np.float32)
    M, N = W.shape
    per_row = N // T
    blocks = np.arange(M * per_row) if blocks is None else np.asarray(blocks, dtype=np.int64)
    soft = np.zeros((blocks.size, T), dtype=np.float64)
    logz = np.zeros(blocks.size, dtype=np.float64)
    dd = None if d is None else np.asarray(d, dtype=np.float32)

    def one(i):
        r, c = divmod(int(blocks[i]), per_row)
        soft[i], logz[i] = bcjr_block(W[r, c * T:(c + 1) * T],
                                      None if dd is None else dd[c * T:(c + 1) * T], C, L,
                                      k, V, T, tau)

    if threads <= 1:
        for i in range(blocks.size):
            one(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(blocks.size)))
    return soft, logz


def hadamard(X, n, sigma=None, inverse=False):
    """Rows of X rotated by R = H_n diag(sigma) / sqrt(n) in chunks of n (inverse: R^T).
    float64 result."""
    f64p = ctypes.POINTER(ctypes.c_double)
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    rows, length = X.shape
    sg = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.float64)
    out = np.empty_like(X)
    lib = _load()
    for r in range(rows):
        xr = np.ascontiguousarray(X[r])
        yr = np.empty(length, dtype=np.float64)
        rc = lib.oracle_hadamard_row(xr.ctypes.data_as(f64p), length, n,
                                     None if sg is None else sg.ctypes.data_as(f64p),
                                     1 if inverse else 0, yr.ctypes.data_as(f64p))
        if rc != 0:
            raise ValueError(f"oracle_hadamard_row failed ({rc})")
        out[r] = yr
    return out


def scale_field(W):
    """(a [M], b [N], Wn [M, N]) in float64 with W = a_r b_c Wn_rc."""
    f64p = ctypes.POINTER(ctypes.c_double)
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, N = W.shape
    a = np.empty(M, dtype=np.float64)
    b = np.empty(N, dtype=np.float64)
    Wn = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_scale_field(_fp(W), M, N, N, a.ctypes.data_as(f64p),
                                    b.ctypes.data_as(f64p), Wn.ctypes.data_as(f64p))
    if rc != 0:
        raise ValueError(f"oracle_scale_field failed ({rc})")
    return a, b, Wn

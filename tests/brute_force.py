"""Independent brute force for tiny trellises (tests only; shares nothing with the
oracle's C code).

Every path (s0, b_1..b_n) is enumerated explicitly and its cost evaluated with the
same fp32 recurrence the encoder is defined by (e = fl(w - c); acc = fmaf(fl(d e), e,
acc)).  Prefix costs are shared between paths that begin alike; that changes nothing
about which paths exist or how each is scored.

`fmaf32` is a vectorized, correctly rounded single-precision fused multiply-add
written from first principles: the float32 product is exact in float64, the sum is
split exactly with Knuth's TwoSum, and the only case where rounding the float64 sum
to float32 can differ from rounding the exact sum (the float64 sum sits exactly on a
float32 rounding midpoint) is resolved by the sign of the TwoSum error.  The test
suite checks it against libm's fmaf.
"""
from __future__ import annotations

import ctypes
import ctypes.util

import numpy as np


def fmaf32(a, b, c):
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b                      # exact: 24 + 24 significant bits
    with np.errstate(invalid="ignore"):
        s = p + c
        bb = s - p                 # TwoSum (Knuth): s + err == p + c exactly
        err = (p - (s - bb)) + (c - bb)
    f = s.astype(np.float32)
    f64 = f.astype(np.float64)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    lo = np.where(f64 > s, dn, f)
    hi = np.where(f64 > s, f, up)
    with np.errstate(invalid="ignore"):
        mid = (lo.astype(np.float64) + hi.astype(np.float64)) * 0.5
    is_mid = (s == mid) & (f64 != s) & np.isfinite(s)
    res = np.where(is_mid & (err > 0), hi, np.where(is_mid & (err < 0), lo, f))
    return res.astype(np.float32)


_libm = None


def libm_fmaf(a: float, b: float, c: float) -> np.float32:
    """libm's fmaf, for checking fmaf32."""
    global _libm
    if _libm is None:
        _libm = ctypes.CDLL(ctypes.util.find_library("m"))
        _libm.fmaf.restype = ctypes.c_float
        _libm.fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
    return np.float32(_libm.fmaf(float(a), float(b), float(c)))


def enumerate_paths(w, d, C, L, k, V, T, fixed_s0=None):
    """All paths of one block.

    Returns (costs float32 [P], states int64 [P, n+1]) where states[:, 0] = s0 and
    states[:, t] = s_t.  Path order: s0 major, then b_1, ..., b_n.
    """
    w = np.asarray(w, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32).reshape(1 << L, V)
    dd = None if d is None else np.asarray(d, dtype=np.float32)
    kv = k * V
    n = T // V
    G = 1 << kv
    mask = (1 << L) - 1
    starts = np.arange(1 << (L - kv), dtype=np.int64)
    if fixed_s0 is not None:
        starts = np.array([fixed_s0], dtype=np.int64)
    states = starts[:, None]
    acc = np.zeros(starts.size, dtype=np.float32)
    for t in range(1, n + 1):
        prev = states[:, -1]
        P = prev.size
        nxt = ((prev[:, None] << kv) | np.arange(G, dtype=np.int64)[None, :]) & mask
        nxt = nxt.reshape(-1)
        a = np.repeat(acc, G)
        for v in range(V):
            i = (t - 1) * V + v
            e = (np.float32(w[i]) - C[nxt, v]).astype(np.float32)
            de = e if dd is None else (np.float32(dd[i]) * e).astype(np.float32)
            a = fmaf32(de, e, a)
        acc = a
        states = np.concatenate([np.repeat(states, G, axis=0), nxt[:, None]], axis=1)
        assert states.shape[0] == P * G
    return acc, states


def path_bits(states, k, V, T):
    """Bitstream words and s0 of one path given its states (for comparisons)."""
    kv = k * V
    n = T // V
    nwords = (k * T + 31) // 32
    words = [0] * nwords
    pos = 0
    for t in range(1, n + 1):
        b = int(states[t]) & ((1 << kv) - 1)
        for i in range(kv - 1, -1, -1):
            bit = (b >> i) & 1
            words[pos // 32] |= bit << (31 - pos % 32)
            pos += 1
    return np.array(words, dtype=np.uint32), int(states[0])


def tie_key(states, L, k, V):
    """(s_n, j_n, j_{n-1}, ..., j_2) with j_t = s_{t-1} >> (L - kV)."""
    kv = k * V
    n = len(states) - 1
    key = [int(states[n])]
    for t in range(n, 1, -1):
        key.append(int(states[t - 1]) >> (L - kv))
    return tuple(key)


def best_path(w, d, C, L, k, V, T, fixed_s0=None):
    """Minimum cost, the optimal path with the smallest tie key, and the second
    smallest cost of the multiset of path costs."""
    costs, states = enumerate_paths(w, d, C, L, k, V, T, fixed_s0)
    order = np.argsort(costs, kind="stable")
    best = costs[order[0]]
    second = costs[order[1]] if costs.size > 1 else np.float32(np.inf)
    cand = np.nonzero(costs == best)[0]
    keys = [tie_key(states[i], L, k, V) for i in cand]
    i_best = cand[int(min(range(len(cand)), key=lambda j: keys[j]))]
    bits, s0 = path_bits(states[i_best], k, V, T)
    return best, second, bits, s0, costs, states

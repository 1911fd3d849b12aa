"""Parity rule between the GPU encoder and the CPU oracle.

Per block: the cost must agree within 1e-5 relative; bitstream and start state must be
identical, except on blocks whose runner-up path (second-smallest fp32 path cost)
lies within 1e-5 relative of the best cost.  An excused block must still carry a path
whose cost, rescored by the oracle, is within 1e-5 relative of the best.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

REL = 1e-5


@dataclass
class ParityReport:
    exact: int = 0
    excused: int = 0
    failures: list = field(default_factory=list)
    max_rel_cost: float = 0.0

    def ok(self) -> bool:
        return not self.failures

    def __str__(self):
        return (f"exact={self.exact} excused={self.excused} failed={len(self.failures)} "
                f"max_rel_cost={self.max_rel_cost:.3g} first={self.failures[:3]}")


def _rel(a, b):
    a = float(a)
    b = float(b)
    if a == b:
        return 0.0
    return abs(a - b) / max(abs(b), 1e-30)


def compare(oracle, W, d, C, L, k, V, T, blocks, g_bits, g_s0, g_cost, threads=8,
            o_result=None) -> ParityReport:
    """g_* are the GPU outputs for the listed blocks (numpy, uint32/float32)."""
    blocks = np.asarray(blocks, dtype=np.int64)
    if o_result is None:
        o_result = oracle.encode_matrix(W, d, C, L, k, V, T, blocks=blocks, threads=threads)
    o_bits, o_s0, o_cost = o_result
    g_bits = np.asarray(g_bits).view(np.uint32).reshape(o_bits.shape)
    g_s0 = np.asarray(g_s0).view(np.uint32).reshape(o_s0.shape)
    g_cost = np.asarray(g_cost, dtype=np.float32).reshape(o_cost.shape)
    rep = ParityReport()
    per_row = W.shape[1] // T
    for i, b in enumerate(blocks):
        rc = _rel(g_cost[i], o_cost[i])
        rep.max_rel_cost = max(rep.max_rel_cost, rc)
        if rc > REL:
            rep.failures.append((int(b), "cost", float(g_cost[i]), float(o_cost[i])))
            continue
        if g_s0[i] == o_s0[i] and np.array_equal(g_bits[i], o_bits[i]):
            rep.exact += 1
            continue
        r, c = divmod(int(b), per_row)
        wb = np.ascontiguousarray(W[r, c * T:(c + 1) * T])
        db = None if d is None else np.ascontiguousarray(d[c * T:(c + 1) * T])
        best, second = oracle.two_best_block(wb, db, C, L, k, V, T)
        gap_ok = (float(second) - float(best)) <= REL * abs(float(best)) if best != 0 \
            else second == 0
        g_path = oracle.path_cost(wb, db, C, L, k, V, T, g_bits[i], int(g_s0[i]))
        if gap_ok and _rel(g_path, best) <= REL and int(g_s0[i]) < (1 << (L - k * V)):
            rep.excused += 1
        else:
            rep.failures.append((int(b), "path", float(best), float(second), float(g_path)))
    return rep

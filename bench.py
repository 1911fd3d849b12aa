"""Throughput of the bitshift-trellis Viterbi encoder on one MI355X.

One step = one tcq_encode call over the whole workload (every coding block: forward
add-compare-select, backpointer store, traceback, packing), inputs resident in HBM.
Default workload: the 2048 x 2048 N(0,1) projection, L=16, k=2, V=1, T=256, d = 1,
65536-entry shuffled Gaussian-quantile codebook.

Prints one JSON line (rank 0).  Alongside the throughput it reports the forward
kernel's roofline -- VALU-bound: algorithmic issue slots per state update (packed fp32
counting one slot) over 256 CUs x 64 slots x 2.4 GHz, the launch timed live with HIP
events on its stream -- and the CPU oracle timed on a bounded sample of the same
workload on this host.  It also times the encode of the other workloads ('workloads';
the 4096 x 4096 weighted one also as 'weighted'), tcq_decode and the fused decode + GEMV
on the encoded matrix, the pre-processing kernels, the soft trellis and the
error-feedback driver.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weights encoded/s (L=16,k=2,T=256 Viterbi) + % VALU peak ACS ops/s"

# MI355X: 256 compute units of 4 SIMDs (16 lanes each), 2.4 GHz peak engine clock.
N_CU = 256
CLOCK_HZ = 2.4e9
HBM_PEAK_GBPS = 8000.0
# VALU issue-slot peak: 256 CUs x 64 lane-slots per clock x 2.4 GHz = 3.93e13 slots/s.  A
# packed-fp32 instruction does two fp32 operations in one slot and an FMA counts as two
# flops, so this is the published 157.3 TFLOP/s fp32 vector rate.
VALU_SLOT_PEAK = N_CU * 64 * CLOCK_HZ
# The same chip counted in non-packed lane operations issued two per SIMD per 4 clocks
# (dual issue from different waves): 7.86e13 lane-ops/s.  Reported as a second view.
VALU_DUAL_ISSUE_PEAK_OPS = 2 * VALU_SLOT_PEAK


def slots_per_state_update(k: int, V: int) -> float:
    """Algorithmic VALU issue slots per state update (one successor at one step), the
    slot model the throughput target is stated in: the branch metric and add take 1.5 V
    packed-fp32 slots (subtract, multiply by d and fused multiply-add per coordinate,
    two lanes per packed slot), and the group compare-select 2 (G - 1) / G slots (G - 1
    minima and G - 1 compares shared by the G = 2^(kV) successors of a group)."""
    G = 2 ** (k * V)
    return 1.5 * V + 2.0 * (G - 1) / G


def valu_ops_per_state_update(k: int, V: int, weighted: bool) -> float:
    """The same work in non-packed lane operations: per coordinate a subtract, a multiply
    by d (weighted only) and a fused multiply-add; per group the tournament of G - 1
    minima and G - 1 compares.  The library is built without packed fp32."""
    G = 2 ** (k * V)
    return V * (3.0 if weighted else 2.0) + 2.0 * (G - 1) / G


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=1, help="index into workloads.WORKLOADS")
    ap.add_argument("--cpu-blocks", type=int, default=1024,
                    help="blocks in the CPU-oracle sample (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="0: min(16, cpu count)")
    ap.add_argument("--gemv-iters", type=int, default=200,
                    help="calls of the fused decode+GEMV timed after the encoder (0: skip)")
    ap.add_argument("--decode-iters", type=int, default=50,
                    help="calls of tcq_decode timed after the encoder (0: skip)")
    ap.add_argument("--also", default="0,2,3,4",
                    help="comma-separated workloads whose encode is also timed (3 or 5 "
                         "steps each, under 'workloads'); workload 2 is also reported as "
                         "'weighted'")
    ap.add_argument("--preprocess-iters", type=int, default=100,
                    help="timed calls of the Hadamard and scale-field kernels (0: skip)")
    ap.add_argument("--bcjr-tau", type=float, default=0.1,
                    help="temperature of the timed soft-trellis run (0: skip)")
    ap.add_argument("--ldlq-workload", type=int, default=2,
                    help="workload whose Hessian drives the timed error-feedback run (-1: skip)")
    ap.add_argument("--ldlq-steps", type=int, default=1)
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES bytes (reference for "
                         "the HBM byte counters) and exit")
    return ap.parse_args()


def log(msg, quiet=False):
    if not quiet:
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()


def measured_traffic(workload_name):
    """HBM bytes per forward launch from the committed rocprofv3 counters, if they were
    taken on the kernel sources as they are now (else None)."""
    import hashlib
    for fn in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not fn.endswith(".counters.json"):
            continue
        with open(os.path.join(ROOT, "profiles", fn)) as f:
            rec = json.load(f)
        if rec.get("workload") != workload_name:
            continue
        h = hashlib.sha256()
        for src in rec["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() == rec["kernel_source_sha256"]:
            return rec["hbm_bytes_per_dispatch"]
    return None


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, W, d, C, nblocks, threads):
    import oracle
    rng = np.random.default_rng(12345)
    blocks = np.sort(rng.choice(w.blocks, size=min(nblocks, w.blocks), replace=False))
    t0 = time.perf_counter()
    oracle.encode_matrix(W, d, C, w.L, w.k, w.V, w.T, blocks=blocks, threads=threads)
    dt = time.perf_counter() - t0
    # one core: the first 32 of those blocks on a single thread
    one = blocks[:32]
    t1 = time.perf_counter()
    oracle.encode_matrix(W, d, C, w.L, w.k, w.V, w.T, blocks=one, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": blocks.size * w.T / dt, "unit": "weights/s", "cores": threads,
            "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": f"{blocks.size} seeded-random blocks of the same workload "
                      f"({blocks.size * w.T} weights), one block per thread at a time, "
                      f"{dt:.2f} s wall",
            "value_1core": one.size * w.T / dt1,
            "sample_1core": f"the first {one.size} of those blocks on one thread, "
                            f"{dt1:.2f} s"}


def gemv_bench(torch, _lib, w, enc, Ct, iters):
    """y = W_hat x on the bitstream the encoder just wrote (batch 1).  Algorithmic bytes:
    the bitstream, the start states, x and y; the codebook gathers hit the L2 cache."""
    g = torch.Generator(device="cpu").manual_seed(77)
    x = torch.randn(w.N, generator=g).to(Ct.device)
    y = torch.empty(w.M, dtype=torch.float32, device=Ct.device)
    stream = torch.cuda.current_stream()

    def call():
        _lib.tcq_decode_gemv(enc.bitstream.data_ptr(), enc.start_state.data_ptr(),
                             Ct.data_ptr(), w.M, w.N, w.L, w.k, w.V, w.T, x.data_ptr(),
                             y.data_ptr(), stream.cuda_stream)

    for _ in range(3):
        call()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / iters
    nbytes = (enc.bitstream.numel() + enc.start_state.numel() + w.N + w.M) * 4
    gbps = nbytes / (us / 1e6) / 1e9
    return {"us_per_call": us, "algorithmic_bytes": nbytes, "achieved_GBps": gbps,
            "frac_hbm": gbps / HBM_PEAK_GBPS, "weights_per_s": w.weights / (us / 1e6)}


def gemv_shapes_bench(torch, _lib, iters):
    """The fused decode + GEMV on the two 8B-class MLP shapes (14336 x 4096 at k = 2,
    V = 2 and 4096 x 14336 at k = 3), on seeded random bitstreams (every stream with
    s_0 < 2^(L-kV) is a trellis path; the decode work does not depend on the path)."""
    out = []
    for M, N, L, k, V, T in ((14336, 4096, 16, 2, 2, 256), (4096, 14336, 16, 3, 1, 256)):
        g = torch.Generator(device="cpu").manual_seed(M + N + k)
        nb = M * (N // T)
        nw = (k * T + 31) // 32
        bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (nb, nw), generator=g,
                             dtype=torch.int32).cuda()
        s0 = torch.randint(0, 1 << (L - k * V), (nb,), generator=g, dtype=torch.int32).cuda()
        C = torch.from_numpy(_lib.tcq_make_codebook(L, V, 3001)).cuda()
        x = torch.randn(N, generator=g).cuda()
        y = torch.empty(M, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()

        def call():
            _lib.tcq_decode_gemv(bits.data_ptr(), s0.data_ptr(), C.data_ptr(), M, N, L, k, V,
                                 T, x.data_ptr(), y.data_ptr(), stream.cuda_stream)

        for _ in range(3):
            call()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / iters
        nbytes = (bits.numel() + s0.numel() + N + M) * 4
        gbps = nbytes / (us / 1e6) / 1e9
        out.append({"shape": f"{M}x{N} L={L} k={k} V={V} T={T}", "us_per_call": us,
                    "algorithmic_bytes": nbytes, "achieved_GBps": gbps,
                    "frac_hbm": gbps / HBM_PEAK_GBPS, "weights_per_s": M * N / (us / 1e6)})
    return out


def ldlq_bench(torch, _lib, wl, index, steps):
    """The error-feedback driver over a whole weighted workload: N/T encodes in sequence
    with the feedback updates between them.  Inputs (W, the block factor U of the
    workload's synthetic Hessian, d) are resident before timing."""
    w = wl.WORKLOADS[index]
    W = torch.from_numpy(wl.make_weights(w)).cuda()
    U_np, d_np = wl.make_ldlq_inputs(w)
    U = torch.from_numpy(U_np).cuda()
    d = torch.from_numpy(d_np).cuda()
    del U_np
    C = torch.from_numpy(_lib.tcq_make_codebook(w.L, w.V, w.codebook_seed)).cuda()
    from trellis_coded_bit_amd import api
    ws = api.Workspace(_lib.tcq_ldlq_workspace_bytes(w.M, w.N, w.L, w.k, w.V, w.T), W.device)
    nb = w.blocks
    bits = torch.empty((nb, api.nwords(w.k, w.T)), dtype=torch.int32, device=W.device)
    s0 = torch.empty(nb, dtype=torch.int32, device=W.device)
    cost = torch.empty(nb, dtype=torch.float32, device=W.device)
    stream = torch.cuda.current_stream()

    def run():
        _lib.tcq_encode_ldlq(W.data_ptr(), w.M, w.N, w.N, U.data_ptr(), w.N, d.data_ptr(),
                             C.data_ptr(), w.L, w.k, w.V, w.T, bits.data_ptr(), s0.data_ptr(),
                             cost.data_ptr(), None, w.N, None, w.N, ws.ptr, ws.nbytes,
                             stream.cuda_stream)

    run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    nblk = w.N // w.T
    fma = w.M * w.T * sum(w.N - (j + 1) * w.T for j in range(nblk))
    return {"workload": w.name, "ms": ms, "weights_per_s": w.weights / (ms / 1e3),
            "column_blocks": nblk, "feedback_fma": fma}


def bcjr_bench(torch, _lib, w, Wt, dt_, Ct, tau, steps):
    """Soft trellis (forward-backward at temperature tau) over the whole bench workload."""
    from trellis_coded_bit_amd import api
    ws = api.Workspace(_lib.tcq_bcjr_workspace_bytes(w.M, w.N, w.L, w.k, w.V, w.T), Wt.device)
    soft = torch.empty((w.M, w.N), dtype=torch.float32, device=Wt.device)
    logz = torch.empty(w.blocks, dtype=torch.float32, device=Wt.device)
    stream = torch.cuda.current_stream()

    def run():
        _lib.tcq_bcjr(Wt.data_ptr(), w.M, w.N, w.N, None if dt_ is None else dt_.data_ptr(),
                      Ct.data_ptr(), w.L, w.k, w.V, w.T, tau, soft.data_ptr(), w.N,
                      logz.data_ptr(), ws.ptr, ws.nbytes, stream.cuda_stream)

    run()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    updates = w.blocks * (w.T // w.V) * (1 << w.L)
    slots = bcjr_slots_per_state(w.k * w.V, w.V)
    rate = updates / (ms / 1e3)
    return {"tau": tau, "ms": ms, "weights_per_s": w.weights / (ms / 1e3),
            "state_updates_per_s_per_pass": rate, "valu_slots_per_state": slots,
            "valu_pct": 100.0 * rate * slots / VALU_DUAL_ISSUE_PEAK_OPS}


def bcjr_slots_per_state(kv, V):
    """Algorithmic VALU issue slots per state for the forward and the backward pass
    together, G = 2^kv states per group, a transcendental (exp2, log2) counted as 2 slots
    (its measured issue cost on gfx950).
    Forward, per state: per coordinate w - c, its square and the fma into the log-weight
    (3V); the group maximum and the sum ((G-1)/G each); the subtraction of the maximum
    and exp2 (1 + 2); per group log2, + maximum, - shift ((2 + 2)/G).
    Backward: the same, plus per coordinate the numerator fma (V), plus per group the
    group weight (+ F, exp2 and the two fmas into numerator and denominator: (1 + 2 + 2)/G)."""
    G = 1 << kv
    fwd = 3 * V + 2 * (G - 1) / G + 3 + 4 / G
    bwd = fwd + V + 5 / G
    return fwd + bwd


def preprocess_bench(torch, _lib, w, Wt, iters):
    """Randomized Hadamard rotation (full row length when it is a power of two <= 4096,
    else chunks of 2048) and the factored scale field, on the bench workload's W.
    Algorithmic bytes: one read and one write of W (8 B per weight)."""
    from trellis_coded_bit_amd import api
    n = w.N if (w.N & (w.N - 1)) == 0 and w.N <= 4096 else 2048
    g = torch.Generator(device="cpu").manual_seed(5)
    sigma = (torch.randint(0, 2, (w.N,), generator=g).float() * 2 - 1).to(Wt.device)
    Y = torch.empty_like(Wt)
    a = torch.empty(w.M, dtype=torch.float32, device=Wt.device)
    b = torch.empty(w.N, dtype=torch.float32, device=Wt.device)
    ws = api.Workspace(_lib.tcq_scale_field_workspace_bytes(w.M, w.N), Wt.device)
    stream = torch.cuda.current_stream()

    def had():
        _lib.tcq_hadamard(Wt.data_ptr(), w.M, w.N, w.N, n, sigma.data_ptr(), False,
                          Y.data_ptr(), w.N, stream.cuda_stream)

    def sf():
        _lib.tcq_scale_field(Wt.data_ptr(), w.M, w.N, w.N, a.data_ptr(), b.data_ptr(),
                             Y.data_ptr(), w.N, ws.ptr, ws.nbytes, stream.cuda_stream)

    out = {}
    for name, fn in (("hadamard", had), ("scale_field", sf)):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        nbytes = 8 * w.weights
        gbps = nbytes / (us / 1e6) / 1e9
        out[name] = {"us": us, "algorithmic_bytes": nbytes, "achieved_GBps": gbps,
                     "frac_hbm": gbps / HBM_PEAK_GBPS}
    out["hadamard"]["n"] = n
    return out


def decode_bench(torch, _lib, w, enc, Ct, iters):
    """tcq_decode of the whole encoded matrix into an M x N buffer.  Algorithmic bytes
    (HBM): 4 B written per weight, plus the bitstream and start states read."""
    out = torch.empty((w.M, w.N), dtype=torch.float32, device=Ct.device)
    stream = torch.cuda.current_stream()

    def call():
        _lib.tcq_decode(enc.bitstream.data_ptr(), enc.start_state.data_ptr(), Ct.data_ptr(),
                        w.M, w.N, w.L, w.k, w.V, w.T, out.data_ptr(), w.N, stream.cuda_stream)

    for _ in range(3):
        call()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / iters
    nbytes = 4 * w.weights + (enc.bitstream.numel() + enc.start_state.numel()) * 4
    gbps = nbytes / (us / 1e6) / 1e9
    return {"us_per_call": us, "algorithmic_bytes": nbytes,
            "bytes_per_weight": nbytes / w.weights, "achieved_GBps": gbps,
            "frac_hbm": gbps / HBM_PEAK_GBPS, "weights_per_s": w.weights / (us / 1e6)}


def decode_shapes_bench(torch, _lib, iters):
    """tcq_decode on the two 8B-class MLP shapes (14336 x 4096 at k = 2, V = 2 and
    4096 x 14336 at k = 3), on seeded random bitstreams, into a dense M x N buffer."""
    out = []
    for M, N, L, k, V, T in ((14336, 4096, 16, 2, 2, 256), (4096, 14336, 16, 3, 1, 256)):
        g = torch.Generator(device="cpu").manual_seed(M + N + k)
        nb = M * (N // T)
        nw = (k * T + 31) // 32
        bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (nb, nw), generator=g,
                             dtype=torch.int32).cuda()
        s0 = torch.randint(0, 1 << (L - k * V), (nb,), generator=g, dtype=torch.int32).cuda()
        C = torch.from_numpy(_lib.tcq_make_codebook(L, V, 3001)).cuda()
        o = torch.empty((M, N), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()

        def call():
            _lib.tcq_decode(bits.data_ptr(), s0.data_ptr(), C.data_ptr(), M, N, L, k, V, T,
                            o.data_ptr(), N, stream.cuda_stream)

        for _ in range(3):
            call()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / iters
        nbytes = 4 * M * N + (bits.numel() + s0.numel()) * 4
        gbps = nbytes / (us / 1e6) / 1e9
        out.append({"shape": f"{M}x{N} L={L} k={k} V={V} T={T}", "us_per_call": us,
                    "algorithmic_bytes": nbytes, "achieved_GBps": gbps,
                    "frac_hbm": gbps / HBM_PEAK_GBPS, "weights_per_s": M * N / (us / 1e6)})
        del bits, s0, o
    return out


def stream_probe_bench(torch, _lib, blocks=2048, super_steps=85):
    """Ceiling of the L = 16, k*V = 2 forward kernel's codebook stream: its codebook loads
    alone (tcq_l16_stream_probe), in bytes per clock per compute unit at 2.4 GHz."""
    from trellis_coded_bit_amd import api
    ws = api.Workspace(_lib.tcq_l16_stream_probe_bytes(blocks), "cuda")
    stream = torch.cuda.current_stream()
    _lib.tcq_l16_stream_probe(blocks, super_steps, ws.ptr, ws.nbytes, stream.cuda_stream,
                              None, None)
    times = []
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)  # torch creates the HIP events at their first record
        b.record(stream)
        _lib.tcq_l16_stream_probe(blocks, super_steps, ws.ptr, ws.nbytes, stream.cuda_stream,
                                  a.cuda_event, b.cuda_event)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = min(times)
    nbytes = blocks * super_steps * 3 * 65536 * 4
    return {"blocks": blocks, "super_steps": super_steps, "ms": ms, "bytes": nbytes,
            "B_per_clk_per_cu": nbytes / (ms / 1e3) / (N_CU * CLOCK_HZ)}


class EncodeRun:
    """One workload's inputs resident on the GPU, its outputs and workspace, and a timed
    loop of tcq_encode_timed calls (the forward launch bracketed by HIP events on the
    launch stream)."""

    def __init__(self, torch, _lib, api, wl, index, quiet):
        self.torch, self._lib = torch, _lib
        w = self.w = wl.WORKLOADS[index]
        log(f"[bench] workload {w.name}: generating inputs", quiet)
        self.W = wl.make_weights(w)
        self.d = wl.make_d(w)
        self.C = _lib.tcq_make_codebook(w.L, w.V, w.codebook_seed)
        dev = torch.device("cuda:0")
        self.Wt = torch.from_numpy(self.W).to(dev)
        self.dt = None if self.d is None else torch.from_numpy(self.d).to(dev)
        self.Ct = torch.from_numpy(self.C).to(dev)
        nb = w.blocks
        self.ws = api.Workspace(_lib.tcq_encode_workspace_bytes(w.M, w.N, w.L, w.k, w.V, w.T),
                                dev)
        self.out = api.Encoded(
            bitstream=torch.empty((nb, api.nwords(w.k, w.T)), dtype=torch.int32, device=dev),
            start_state=torch.empty(nb, dtype=torch.int32, device=dev),
            cost=torch.empty(nb, dtype=torch.float32, device=dev), recon=None)

    def step(self, e0=None, e1=None):
        w, t = self.w, self.torch
        self._lib.tcq_encode_timed(
            self.Wt.data_ptr(), w.M, w.N, w.N, None if self.dt is None else self.dt.data_ptr(),
            self.Ct.data_ptr(), w.L, w.k, w.V, w.T, self.out.bitstream.data_ptr(),
            self.out.start_state.data_ptr(), self.out.cost.data_ptr(), None, w.N, self.ws.ptr,
            self.ws.nbytes, t.cuda.current_stream().cuda_stream, e0, e1)

    def timed(self, steps, warmup):
        """(ms per step by the host clock, forward-launch ms of every timed step)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:  # torch creates its events lazily, at the first record
            a.record(stream)
            b.record(stream)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in ev:
            self.step(a.cuda_event, b.cuda_event)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        return ms, [a.elapsed_time(b) for a, b in ev]

    def summary(self, ms_per_step, acs):
        """Throughput and the forward kernel's rates for one timed run."""
        w = self.w
        acs_ms = float(np.mean(acs))
        updates = w.blocks * (w.T // w.V) * (1 << w.L)
        rate = updates / (acs_ms / 1e3)
        slots = slots_per_state_update(w.k, w.V)
        ops = valu_ops_per_state_update(w.k, w.V, self.d is not None)
        bp_bytes = w.blocks * (w.T // w.V) * (1 << (w.L - w.k * w.V)) * (w.k * w.V) / 8
        # Every state update reads its successor's V codebook values (fp32) from the
        # L2-resident codebook copies: this stream, not HBM, bounds the register-resident
        # forward kernels in practice.
        cb_bytes = updates * 4 * w.V
        return {"workload": w.name, "ms_per_step": ms_per_step,
                "weights_per_s": w.weights / (ms_per_step / 1e3),
                "kernel_ms": acs_ms, "kernel_ms_each": acs,
                "state_updates_per_launch": updates, "state_updates_per_s": rate,
                "slots_per_update": slots,
                "valu_pct_slot_model": 100.0 * rate * slots / VALU_SLOT_PEAK,
                "valu_ops_per_update": ops,
                "valu_pct_dual_issue_ops": 100.0 * rate * ops / VALU_DUAL_ISSUE_PEAK_OPS,
                "bp_write_GBps": bp_bytes / (acs_ms / 1e3) / 1e9,
                "bp_pct_hbm": 100.0 * bp_bytes / (acs_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                "codebook_l2_B_per_clk_per_cu": cb_bytes / (acs_ms / 1e3) / (N_CU * CLOCK_HZ),
                "share_of_step": acs_ms / ms_per_step}

    def free(self):
        del self.Wt, self.dt, self.Ct, self.ws, self.out
        self.torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every coding block is independent; see the sharding note in the docs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from trellis_coded_bit_amd import _lib, api
    from trellis_coded_bit_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}))
        return
    _lib.load()  # fail loudly if the HIP library is missing
    run = EncodeRun(torch, _lib, api, wl, args.workload, args.quiet)
    w = run.w
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps", args.quiet)
    ms_per_step, acs = run.timed(args.steps, args.warmup)
    main_sum = run.summary(ms_per_step, acs)
    acs_ms = main_sum["kernel_ms"]
    # roofline of the forward kernel, in the slot model: algorithmic slots per state
    # update x updates per launch / the launch's duration, against 3.93e13 slots/s
    achieved = main_sum["state_updates_per_s"] * main_sum["slots_per_update"] / 1e12
    peak = VALU_SLOT_PEAK / 1e12

    result = {
        "metric": METRIC,
        "value": main_sum["weights_per_s"],
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "L": w.L, "k": w.k, "V": w.V,
                   "T": w.T, "d": "weighted (LDL diagonal)" if run.d is not None else "1 (NULL)",
                   "codebook": f"2^{w.L} shuffled Gaussian quantiles, seed {w.codebook_seed}"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak,
                     "unit": "Tslot/s", "frac": achieved / peak,
                     "model": "VALU issue slots: 1.5 V + 2 (G - 1) / G per state update "
                              "(packed fp32 = 1 slot), peak 256 CU x 64 x 2.4 GHz",
                     "traffic": measured_traffic(w.name)},
        "acs": main_sum,
    }
    if args.gemv_iters > 0:
        log(f"[bench] fused decode+GEMV on the encoded matrix, {args.gemv_iters} calls",
            args.quiet)
        result["decode_gemv"] = gemv_bench(torch, _lib, w, run.out, run.Ct, args.gemv_iters)
    if args.gemv_iters > 0:
        log("[bench] fused decode+GEMV on the 8B-class MLP shapes", args.quiet)
        result["decode_gemv_shapes"] = gemv_shapes_bench(torch, _lib, max(10, args.gemv_iters // 2))
    if args.decode_iters > 0:
        log(f"[bench] decode of the encoded matrix, {args.decode_iters} calls", args.quiet)
        result["decode"] = decode_bench(torch, _lib, w, run.out, run.Ct, args.decode_iters)
        log("[bench] decode on the 8B-class MLP shapes", args.quiet)
        result["decode_shapes"] = decode_shapes_bench(torch, _lib, max(5, args.decode_iters // 5))
    if w.L == 16 and w.k * w.V == 2:
        log("[bench] codebook-stream probe of the forward kernel", args.quiet)
        probe = stream_probe_bench(torch, _lib)
        probe["forward_kernel_share"] = (main_sum["codebook_l2_B_per_clk_per_cu"] /
                                         probe["B_per_clk_per_cu"])
        result["acs"]["codebook_stream_probe"] = probe
    if args.preprocess_iters > 0:
        log("[bench] pre-processing kernels", args.quiet)
        result["preprocess"] = preprocess_bench(torch, _lib, w, run.Wt, args.preprocess_iters)
    if args.bcjr_tau > 0:
        log(f"[bench] soft trellis at tau={args.bcjr_tau}", args.quiet)
        result["bcjr"] = bcjr_bench(torch, _lib, w, run.Wt, run.dt, run.Ct, args.bcjr_tau, 1)
    W, d, C = run.W, run.d, run.C
    run.free()
    others = [int(x) for x in args.also.split(",") if x.strip() != ""]
    for idx in others:
        if idx == args.workload:
            continue
        o = EncodeRun(torch, _lib, api, wl, idx, args.quiet)
        steps = 3 if o.w.weights > 20e6 else 5
        log(f"[bench] workload {o.w.name}: warmup 1, timing {steps} steps", args.quiet)
        oms, oacs = o.timed(steps, 1)
        entry = o.summary(oms, oacs)
        entry["steps"] = steps
        if args.preprocess_iters > 0 and o.w.index == 2:
            log("[bench] pre-processing kernels on the 4096 x 4096 weights", args.quiet)
            entry["preprocess"] = preprocess_bench(torch, _lib, o.w, o.Wt,
                                                   args.preprocess_iters)
        o.free()
        result.setdefault("workloads", {})[o.w.name] = entry
        if o.w.index == 2:
            result["weighted"] = entry
    if args.ldlq_workload >= 0:
        log(f"[bench] error-feedback driver on workload {args.ldlq_workload}", args.quiet)
        result["ldlq"] = ldlq_bench(torch, _lib, wl, args.ldlq_workload, args.ldlq_steps)
    if args.cpu_blocks > 0:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        log(f"[bench] cpu oracle on {args.cpu_blocks} blocks, {threads} threads", args.quiet)
        result["cpu_baseline"] = cpu_baseline(w, W, d, C, args.cpu_blocks, threads)
    print(json.dumps(result))
    sys.stdout.flush()


if __name__ == "__main__":
    main()

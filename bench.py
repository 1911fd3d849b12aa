"""Throughput of the bitshift-trellis Viterbi encoder on one MI355X.

One step = one tcq_encode call over the whole workload (every coding block: forward
add-compare-select, backpointer store, traceback, packing), inputs resident in HBM.
Default workload: the 2048 x 2048 N(0,1) projection, L=16, k=2, V=1, T=256, d = 1,
65536-entry shuffled Gaussian-quantile codebook.

Prints one JSON line (rank 0).  Alongside the throughput it reports the forward
kernel's roofline (VALU-bound: algorithmic VALU operations per state update over the
chip's VALU issue rate, timed live with HIP events around the forward launch) and the
CPU oracle timed on a bounded sample of the same workload on this host.
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

# MI355X: 256 compute units of 4 SIMDs, 2.4 GHz peak engine clock.  A SIMD issues up to
# two wave64 VALU instructions (from different waves) every 4 clocks: 128 VALU lane-ops
# per clock per CU, non-packed.  This is the published fp32 vector rate (157.3 TFLOP/s)
# with an FMA counted as one op instead of two.  (Not every instruction pairs: v_min3 and
# other 3-source integer ops issue one per 4 clocks.)
N_CU = 256
LANES_PER_CU_CLK = 128
CLOCK_HZ = 2.4e9
VALU_PEAK_OPS = N_CU * LANES_PER_CU_CLK * CLOCK_HZ  # 7.86e13 lane-ops/s
HBM_PEAK_GBPS = 8000.0


def valu_ops_per_state_update(k: int, V: int, weighted: bool) -> float:
    """Algorithmic VALU lane-ops per state update (one successor at one step):
    per coordinate a subtract, a multiply by d (weighted only) and a fused multiply-add;
    per group of G = 2^(kV) predecessors a tournament of G-1 minima and G-1 compares
    (for the lowest-index argmin), shared by the group's G successors."""
    G = 2 ** (k * V)
    return V * (3.0 if weighted else 2.0) + 2.0 * (G - 1) / G


def packed_slot_model_pct(updates_per_s: float, k: int, V: int) -> float:
    """The slot model the target is stated in: per state update 1.5 V packed-fp32 slots
    for the branch metric and add, plus 2 (G - 1) / G for the group compare-select,
    against 256 CUs x 64 slots per clock x 2.4 GHz (3.93e13 slots/s).  Reported next to
    the roofline, which is against the dual-issue peak and counts non-packed operations."""
    G = 2 ** (k * V)
    slots = 1.5 * V + 2.0 * (G - 1) / G
    return 100.0 * updates_per_s * slots / (N_CU * 64 * CLOCK_HZ)


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
            "valu_pct": 100.0 * rate * slots / VALU_PEAK_OPS}


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
    w = wl.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: generating inputs", args.quiet)
    W = wl.make_weights(w)
    d = wl.make_d(w)
    C = _lib.tcq_make_codebook(w.L, w.V, w.codebook_seed)
    dev = torch.device("cuda:0")
    Wt = torch.from_numpy(W).to(dev)
    dt_ = None if d is None else torch.from_numpy(d).to(dev)
    Ct = torch.from_numpy(C).to(dev)
    nb = w.blocks
    ws_bytes = _lib.tcq_encode_workspace_bytes(w.M, w.N, w.L, w.k, w.V, w.T)
    ws = api.Workspace(ws_bytes, dev)
    out = api.Encoded(
        bitstream=torch.empty((nb, api.nwords(w.k, w.T)), dtype=torch.int32, device=dev),
        start_state=torch.empty(nb, dtype=torch.int32, device=dev),
        cost=torch.empty(nb, dtype=torch.float32, device=dev), recon=None)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:  # torch creates its events lazily, at the first record
        a.record(stream)
        b.record(stream)

    def step(i=None):
        e0, e1 = (None, None) if i is None else (ev[i][0].cuda_event, ev[i][1].cuda_event)
        _lib.tcq_encode_timed(Wt.data_ptr(), w.M, w.N, w.N,
                              None if dt_ is None else dt_.data_ptr(), Ct.data_ptr(), w.L,
                              w.k, w.V, w.T, out.bitstream.data_ptr(),
                              out.start_state.data_ptr(), out.cost.data_ptr(), None, w.N,
                              ws.ptr, ws.nbytes, stream.cuda_stream, e0, e1)

    log(f"[bench] warmup {args.warmup}", args.quiet)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps", args.quiet)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    acs_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    weights_per_s = w.weights / (ms_per_step / 1e3)

    updates_per_launch = nb * (w.T // w.V) * (1 << w.L)
    ops = valu_ops_per_state_update(w.k, w.V, d is not None)
    acs_ops_per_s = updates_per_launch / (acs_ms / 1e3)
    achieved_tops = acs_ops_per_s * ops / 1e12
    peak_tops = VALU_PEAK_OPS / 1e12
    bp_bytes = nb * (w.T // w.V) * (1 << (w.L - w.k * w.V)) * (w.k * w.V) / 8
    bp_gbps = bp_bytes / (acs_ms / 1e3) / 1e9
    # Every state update reads its successor's V codebook values (fp32) from L2: the
    # register-resident forward kernels stream 4 V bytes per update from the L2-resident
    # codebook copies, and this stream, not HBM, is what bounds them in practice.
    cb_bytes = updates_per_launch * 4 * w.V
    cb_b_per_clk_cu = cb_bytes / (acs_ms / 1e3) / (N_CU * CLOCK_HZ)

    result = {
        "metric": METRIC,
        "value": weights_per_s,
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
                   "T": w.T, "d": "weighted (LDL diagonal)" if d is not None else "1 (NULL)",
                   "codebook": f"2^{w.L} shuffled Gaussian quantiles, seed {w.codebook_seed}"},
        "roofline": {"bound": "alu", "achieved": achieved_tops, "peak": peak_tops,
                     "unit": "TOP/s", "frac": achieved_tops / peak_tops,
                     "traffic": measured_traffic(w.name)},
        "acs": {"kernel_ms": acs_ms, "state_updates_per_s": acs_ops_per_s,
                "valu_ops_per_update": ops, "valu_pct": 100.0 * achieved_tops / peak_tops,
                "valu_pct_packed_slot_model": packed_slot_model_pct(acs_ops_per_s, w.k, w.V),
                "bp_write_GBps": bp_gbps, "bp_pct_hbm": 100.0 * bp_gbps / HBM_PEAK_GBPS,
                "codebook_l2_bytes": cb_bytes, "codebook_l2_B_per_clk_per_cu": cb_b_per_clk_cu,
                "share_of_step": acs_ms / ms_per_step},
    }
    if args.gemv_iters > 0:
        log(f"[bench] fused decode+GEMV on the encoded matrix, {args.gemv_iters} calls",
            args.quiet)
        result["decode_gemv"] = gemv_bench(torch, _lib, w, out, Ct, args.gemv_iters)
    if args.preprocess_iters > 0:
        log("[bench] pre-processing kernels", args.quiet)
        result["preprocess"] = preprocess_bench(torch, _lib, w, Wt, args.preprocess_iters)
    if args.bcjr_tau > 0:
        log(f"[bench] soft trellis at tau={args.bcjr_tau}", args.quiet)
        result["bcjr"] = bcjr_bench(torch, _lib, w, Wt, dt_, Ct, args.bcjr_tau, 1)
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

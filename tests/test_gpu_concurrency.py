"""Several host threads, each on its own HIP stream, call the library at the same time:
the results are bitwise those of the same calls made one after another.  (Apart from the
per-thread error string, the library keeps only a process-wide cache of kernel attributes,
which is locked.)"""
import sys
import threading

import numpy as np
import pytest

from trellis_coded_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import api  # noqa: E402

L, K, V, T = 16, 2, 1, 256
M, N = 6, 1024  # 24 coding blocks per problem
THREADS = 4


def _problem(seed):
    W, d = wl.random_small(seed, M, N, weighted=True)
    x = np.random.default_rng(seed).standard_normal(N).astype(np.float32)
    return W, d, x


def _run(C, W, d, x):
    out = api.encode(torch.from_numpy(W).cuda(), torch.from_numpy(d).cuda(), C, L, K, V, T,
                     recon=False)
    y = api.decode_gemv(out.bitstream, out.start_state, C, torch.from_numpy(x).cuda(), M, N,
                        L, K, V, T)
    return out.bitstream, out.start_state, out.cost, y


def test_threads_on_own_streams_match_sequential():
    sys.stdout.write("concurrency: 4 host threads, encode + decode-GEMV\n")
    sys.stdout.flush()
    C = api.make_codebook(L, V, 3001)
    probs = [_problem(100 + i) for i in range(THREADS)]
    ref = []
    for P in probs:
        r = _run(C, *P)
        torch.cuda.synchronize()
        ref.append([t.cpu().numpy() for t in r])
    res = [None] * THREADS
    errs = []
    start = threading.Barrier(THREADS)

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait(timeout=60)
                r = _run(C, *probs[i])
                s.synchronize()
                res[i] = [t.cpu().numpy() for t in r]
        except Exception as e:  # reported below
            errs.append(e)

    ths = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in ths:
        t.start()
    for t in ths:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ths)
    assert not errs, errs
    for i in range(THREADS):
        for got, want in zip(res[i], ref[i]):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))

"""Full-size workloads on the GPU, in the launch configuration bench.py times (whole
matrix, recommended workspace), checked against the oracle under the bar of parity.py:

- the 2048 x 2048 and the 4096 x 4096 weighted workloads: every block (the latter in
  four chunks of 16384 blocks, so that progress is printed as it goes);
- the 4096 x 14336 (k = 3) and 14336 x 4096 (V = 2) workloads: a seeded uniform sample
  of 8192 blocks plus every block of the first and the last row, or every block (14
  chunks each, about 7 minutes of oracle time on 16 threads) for the workloads listed
  in TCQ_TEST_FULL_WORKLOADS (e.g. "3,4").

Each case prints its exact / excused / failed block counts."""
import os
import sys
import time

import numpy as np
import pytest

import parity
from trellis_coded_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import _lib, api  # noqa: E402

THREADS = min(16, os.cpu_count() or 1)
SAMPLE = int(os.environ.get("TCQ_TEST_SAMPLE_BLOCKS", "8192"))
CHUNK = 16384

FULL = {int(x) for x in os.environ.get("TCQ_TEST_FULL_WORKLOADS", "").split(",") if x.strip()}

# (workload index, chunk): chunk i of a fully checked workload covers blocks
# [i * CHUNK, (i + 1) * CHUNK); chunk -1 is the sample of a sampled workload.
CASES = [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3)]
for _i in (3, 4):
    if _i in FULL:
        _n = wl.WORKLOADS[_i].blocks
        CASES += [(_i, c) for c in range((_n + CHUNK - 1) // CHUNK)]
    else:
        CASES.append((_i, -1))

_cache = {}


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _encoded(oracle_lib, index):
    """Inputs and GPU outputs of one workload, computed once per workload."""
    if index in _cache:
        return _cache[index]
    _cache.clear()  # one workload's inputs at a time
    w = wl.WORKLOADS[index]
    t0 = time.time()
    _say(f"workload {w.name}: generating inputs")
    W = wl.make_weights(w)
    d = wl.make_d(w)
    C = _lib.tcq_make_codebook(w.L, w.V, w.codebook_seed)
    assert np.array_equal(C, oracle_lib.make_codebook(w.L, w.V, w.codebook_seed))
    _say(f"  inputs ready in {time.time() - t0:.1f}s; encoding {w.blocks} blocks on the GPU")
    dev = torch.device("cuda:0")
    out = api.encode(torch.from_numpy(W).to(dev),
                     None if d is None else torch.from_numpy(d).to(dev),
                     torch.from_numpy(C).to(dev), w.L, w.k, w.V, w.T)
    torch.cuda.synchronize()
    res = dict(w=w, W=W, d=d, C=C,
               bits=out.bitstream.cpu().numpy().view(np.uint32),
               s0=out.start_state.cpu().numpy().view(np.uint32),
               cost=out.cost.cpu().numpy())
    del out
    torch.cuda.empty_cache()
    _say(f"  GPU done at {time.time() - t0:.1f}s")
    _cache[index] = res
    return res


@pytest.mark.timeout(900)
@pytest.mark.parametrize("index,chunk", CASES, ids=[f"w{i}-{'sample' if c < 0 else c}"
                                                    for i, c in CASES])
def test_workload_parity(oracle_lib, index, chunk):
    e = _encoded(oracle_lib, index)
    w = e["w"]
    if chunk < 0:
        blocks = wl.sample_blocks(w, SAMPLE, seed=100 + index)
        what = f"sample of {blocks.size} blocks (incl. rows 0 and {w.M - 1})"
    else:
        blocks = np.arange(chunk * CHUNK, min((chunk + 1) * CHUNK, w.blocks))
        what = f"blocks {blocks[0]}..{blocks[-1]} of {w.blocks}"
    t0 = time.time()
    rep = parity.compare(oracle_lib, e["W"], e["d"], e["C"], w.L, w.k, w.V, w.T, blocks,
                         e["bits"][blocks], e["s0"][blocks], e["cost"][blocks],
                         threads=THREADS)
    _say(f"  {w.name}: {what}: exact={rep.exact} excused={rep.excused} "
         f"failed={len(rep.failures)} ({time.time() - t0:.1f}s, {THREADS} threads)")
    assert rep.ok(), str(rep)
    if chunk <= 0:
        # every block of the launch: finite costs and start states in range
        assert np.all(np.isfinite(e["cost"]))
        assert np.all(e["s0"] < (1 << (w.L - w.k * w.V)))

"""tcq_encode_noalloc, the encoder entry point for callers that cannot allocate device
memory, against tcq_encode with a torch-allocated workspace, through the C ABI.

Bitstreams, start states, costs and reconstructions must be identical bit for bit, on two
calls in a row, the second with a smaller input: the library's scratch array keeps what the
first call left in it.  The first call of each case has more blocks than one batch of the
scratch holds, so it also runs the batching.
"""
import sys

import numpy as np
import pytest

from trellis_coded_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import _lib, api  # noqa: E402


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _noalloc(W, d, C, L, k, V, T, recon):
    M, N = W.shape
    nb = M * (N // T)
    bits = torch.full((nb, api.nwords(k, T)), -1, dtype=torch.int32, device="cuda")
    s0 = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    cost = torch.full((nb,), -1.0, dtype=torch.float32, device="cuda")
    rec = torch.full((M, N), -1.0, dtype=torch.float32, device="cuda") if recon else None
    _lib.tcq_encode_noalloc(W.data_ptr(), M, N, W.stride(0),
                            None if d is None else d.data_ptr(), C.data_ptr(), L, k, V, T,
                            bits.data_ptr(), s0.data_ptr(), cost.data_ptr(),
                            None if rec is None else rec.data_ptr(), N,
                            torch.cuda.current_stream().cuda_stream)
    return bits, s0, cost, rec


CASES = [
    # L, k, V, T, (M, N) of the first call, (M, N) of the second, weighted
    (16, 2, 1, 256, (80, 1024), (3, 512), False),   # 320 blocks: two batches of <= 255
    (16, 2, 1, 256, (66, 1024), (1, 256), True),
    (16, 3, 1, 256, (40, 2048), (2, 256), True),    # 320 blocks, k = 3 kernel
    (16, 2, 2, 256, (70, 1024), (5, 256), True),    # k*V = 4 kernel
    (10, 2, 1, 64, (20, 512), (3, 128), False),     # generic kernel
]


@pytest.mark.parametrize("L,k,V,T,first,second,weighted", CASES)
def test_noalloc_matches_encode(oracle_lib, L, k, V, T, first, second, weighted):
    C = torch.from_numpy(oracle_lib.make_codebook(L, V, 41)).cuda()
    for call, (M, N) in enumerate((first, second)):
        _say(f"noalloc L={L} k={k} V={V} T={T} call {call}: M={M} N={N} weighted={weighted}")
        Wn, dn = wl.random_small(77 + 10 * call + L + k, M, N, weighted)
        W = torch.from_numpy(Wn).cuda()
        d = None if dn is None else torch.from_numpy(dn).cuda()
        ref = api.encode(W, d, C, L, k, V, T, recon=True)
        bits, s0, cost, rec = _noalloc(W, d, C, L, k, V, T, recon=True)
        torch.cuda.synchronize()
        assert torch.equal(bits, ref.bitstream)
        assert torch.equal(s0, ref.start_state)
        assert torch.equal(cost.view(torch.int32), ref.cost.view(torch.int32))
        assert torch.equal(rec.view(torch.int32), ref.recon.view(torch.int32))


def test_noalloc_rejects_bad_arguments():
    with pytest.raises(_lib.TcqError) as e:
        _lib.tcq_encode_noalloc(0, 2, 100, 100, None, 0, 16, 2, 1, 256, 0, 0, 0, None, 100, None)
    assert e.value.status == _lib.TCQ_EINVAL
    assert "tcq_encode_noalloc" in str(e.value)

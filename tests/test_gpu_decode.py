"""tcq_decode (the reconstruction W_hat of a bitstream) vs. the oracle's decode, bit for bit.

Decoding copies codebook rows, so the bar is identity of every output bit pattern.  Inputs
are seeded random bitstreams with start states below 2^(L-kV) (every such stream is a path
of the trellis); nothing comes from the GPU encoder.  The cases cover the LDS-staged unit
kernel for every (k*V, V) it is built for, with 1 to 8 codebook parts, several tiles per
workgroup and a ragged last tile, both store widths (row strides with and without 16-byte
alignment), codebooks that do not start on 16 bytes, and the per-block kernel that takes
every other shape; the codebook carries
-0.0, +0.0, a denormal and infinities, which must come out unchanged.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

from trellis_coded_bit_amd import _lib, api  # noqa: E402


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _streams(rng, nb, L, k, V, T):
    nw = (k * T + 31) // 32
    bits = rng.integers(0, 1 << 32, size=(nb, nw), dtype=np.uint64).astype(np.uint32)
    tail = k * T % 32
    if tail:
        bits[:, -1] &= np.uint32(((1 << tail) - 1) << (32 - tail))
    s0 = rng.integers(0, 1 << (L - k * V), size=nb, dtype=np.uint64).astype(np.uint32)
    return bits, s0


def _codebook(oracle_lib, L, V, seed):
    C = oracle_lib.make_codebook(L, V, seed).copy()
    flat = C.reshape(-1)
    special = np.array([0x80000000, 0x00000000, 0x00000001, 0x7F800000, 0xFF800000],
                       dtype=np.uint32).view(np.float32)
    flat[:special.size] = special
    return C


def _gpu_decode(bits, s0, C, M, N, L, k, V, T, ldo=None, c_shift=0):
    """c_shift > 0 places the codebook c_shift floats into its allocation (not 16-byte
    aligned for c_shift = 1, 2, 3)."""
    ldo = N if ldo is None else ldo
    bt = torch.from_numpy(bits.view(np.int32)).cuda()
    st = torch.from_numpy(s0.view(np.int32)).cuda()
    flat = torch.from_numpy(np.ascontiguousarray(C).reshape(-1))
    Cbuf = torch.full((flat.numel() + c_shift,), float("nan"), dtype=torch.float32)
    Cbuf[c_shift:] = flat
    Ct = Cbuf.cuda()[c_shift:]
    out = torch.full((max(M, 1), ldo), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.tcq_decode(bt.data_ptr(), st.data_ptr(), Ct.data_ptr(), M, N, L, k, V, T,
                    out.data_ptr(), ldo, stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # L, k, V, T, M, N, ldo (None: N)
    (16, 2, 1, 256, 64, 2048, None),     # k*V = 2, two parts
    (16, 2, 1, 256, 33, 1024, 1027),     # unaligned row stride: 4-byte stores
    (16, 2, 1, 256, 17, 768, 772),       # aligned stride past N: 16-byte stores
    (16, 2, 2, 256, 40, 1024, None),     # k*V = 4, V = 2: four parts
    (16, 3, 1, 256, 24, 1536, None),     # three-word units
    (16, 1, 1, 128, 20, 512, None),      # k*V = 1: one unit of 32 steps per word
    (16, 1, 2, 128, 12, 512, None),      # k*V = 2, V = 2
    (16, 1, 4, 128, 10, 256, None),      # k*V = 4, V = 4: eight parts
    (16, 2, 4, 256, 8, 512, 514),        # k*V = 8, V = 4, 8-byte aligned stride
    (14, 4, 1, 64, 30, 640, None),       # k*V = 4, one part
    (12, 3, 2, 96, 9, 384, None),        # k*V = 6, V = 2
    (12, 8, 1, 32, 11, 320, None),       # k*V = 8, units of four steps
    (10, 6, 1, 48, 7, 192, 193),         # k*V = 6, V = 1
    (15, 4, 2, 64, 5, 256, None),        # k*V = 8, V = 2
    (9, 2, 1, 100, 6, 300, None),        # block not a whole number of units: per-block kernel
    (8, 3, 1, 10, 4, 40, 41),            # 30-bit blocks: per-block kernel
    # tables smaller than one wave's 64-float4 chunk of the part copy (lanes past the
    # table load zeros) and exactly one chunk
    (6, 2, 1, 64, 9, 256, None),         # 16 float4
    (5, 1, 4, 32, 6, 128, None),         # 32 float4, V = 4
    (7, 1, 2, 64, 5, 256, None),         # 64 float4
]


@pytest.mark.parametrize("L,k,V,T,M,N,ldo", CASES)
def test_decode_bitwise(oracle_lib, L, k, V, T, M, N, ldo):
    _say(f"decode L={L} k={k} V={V} T={T} M={M} N={N} ldo={ldo}")
    rng = np.random.default_rng(L * 1000 + k * 100 + V * 10 + M)
    C = _codebook(oracle_lib, L, V, 21 + L)
    bits, s0 = _streams(rng, M * (N // T), L, k, V, T)
    ref = oracle_lib.decode_matrix(bits, s0, C, M, N, L, k, V, T)
    out = _gpu_decode(bits, s0, C, M, N, L, k, V, T, ldo)
    assert np.array_equal(out[:, :N].view(np.uint32), ref.view(np.uint32))
    if ldo is not None and ldo > N:
        assert np.all(np.isnan(out[:, N:])), "decode wrote past N"


@pytest.mark.parametrize("L,k,V,T,M,N,ldo,c_shift", [
    (16, 2, 1, 256, 64, 2048, None, 1),   # dense rows, two parts
    (16, 2, 2, 256, 40, 1024, None, 2),   # dense rows, four parts
    (16, 3, 1, 256, 24, 1536, None, 3),   # dense rows, three-word units
    (16, 2, 1, 256, 33, 1024, 1027, 1),   # strided rows
    (7, 1, 2, 64, 5, 256, None, 1),       # one part smaller than the workgroup
])
def test_decode_unaligned_codebook(oracle_lib, L, k, V, T, M, N, ldo, c_shift):
    """A codebook that does not start on 16 bytes is copied into LDS float by float."""
    _say(f"decode L={L} k={k} V={V} T={T} M={M} N={N} ldo={ldo} codebook +{c_shift} floats")
    rng = np.random.default_rng(L * 1000 + k * 100 + V * 10 + M + 7 * c_shift)
    C = _codebook(oracle_lib, L, V, 77 + L)
    bits, s0 = _streams(rng, M * (N // T), L, k, V, T)
    ref = oracle_lib.decode_matrix(bits, s0, C, M, N, L, k, V, T)
    out = _gpu_decode(bits, s0, C, M, N, L, k, V, T, ldo, c_shift)
    assert np.array_equal(out[:, :N].view(np.uint32), ref.view(np.uint32))
    if ldo is not None and ldo > N:
        assert np.all(np.isnan(out[:, N:])), "decode wrote past N"


def test_decode_many_tiles_per_workgroup(oracle_lib):
    """8192 x 4096 at k = 2: 2^21 units, several tiles per workgroup and a ragged last one."""
    L, k, V, T, M, N = 16, 2, 1, 256, 8192, 4096
    _say(f"decode L={L} k={k} V={V} T={T} M={M} N={N}")
    rng = np.random.default_rng(8192)
    C = _codebook(oracle_lib, L, V, 3001)
    bits, s0 = _streams(rng, M * (N // T), L, k, V, T)
    out = _gpu_decode(bits, s0, C, M, N, L, k, V, T)
    ref = oracle_lib.decode_matrix(bits, s0, C, M, N, L, k, V, T)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_decode_full_size_sampled_rows(oracle_lib):
    """14336 x 4096 at k = 2, V = 2 (the 8B-class MLP shape): rows 0, M-1 and 62 seeded rows
    are decoded by the oracle and compared bit for bit."""
    L, k, V, T, M, N = 16, 2, 2, 256, 14336, 4096
    _say(f"decode L={L} k={k} V={V} T={T} M={M} N={N} (sampled rows)")
    rng = np.random.default_rng(14336)
    C = _codebook(oracle_lib, L, V, 3001)
    per_row = N // T
    bits, s0 = _streams(rng, M * per_row, L, k, V, T)
    out = _gpu_decode(bits, s0, C, M, N, L, k, V, T)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
    sel = (rows[:, None] * per_row + np.arange(per_row)[None, :]).reshape(-1)
    ref = oracle_lib.decode_matrix(bits[sel], s0[sel], C, rows.size, N, L, k, V, T)
    assert np.array_equal(out[rows].view(np.uint32), ref.view(np.uint32))


def test_decode_empty(oracle_lib):
    """Empty shapes launch nothing and return."""
    L, k, V, T = 16, 2, 1, 256
    Ct = torch.from_numpy(oracle_lib.make_codebook(L, V, 1)).cuda()
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    out = api.decode(empty, empty, Ct, 0, 512, L, k, V, T)
    assert out.shape == (0, 512)
    out = api.decode(empty, empty, Ct, 4, 0, L, k, V, T)
    assert out.shape == (4, 0)
    torch.cuda.synchronize()

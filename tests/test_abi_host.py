"""Host-side checks of libtcq: it loads, exports every symbol the header declares, its
codebook builder agrees bit for bit with the oracle's, and argument checks reject bad
calls before anything reaches a GPU (no device work is issued by these tests)."""
import os
import re

import numpy as np
import pytest

import trellis_coded_bit_amd as tcq
from trellis_coded_bit_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000001000  # never dereferenced: every call below fails validation first


def _declared():
    with open(os.path.join(ROOT, "include", "tcq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(tcq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_declared_symbols():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
    assert tcq.tcq_version() >= 100


@pytest.mark.parametrize("L,V,seed", [(1, 1, 0), (2, 1, 42), (8, 1, 3000), (12, 1, 9),
                                      (16, 1, 3001), (16, 2, 3004), (9, 2, 5), (10, 3, 77),
                                      (16, 4, 1)])
def test_codebook_matches_oracle(oracle_lib, L, V, seed):
    lib_cb = tcq.tcq_make_codebook(L, V, seed)
    ora_cb = oracle_lib.make_codebook(L, V, seed)
    assert lib_cb.shape == ora_cb.shape
    assert np.array_equal(lib_cb.view(np.uint32), ora_cb.view(np.uint32))


def test_codebook_rejects_bad_args():
    for L, V in [(0, 1), (25, 1), (4, 0), (3, 4), (16, 9)]:
        with pytest.raises(tcq.TcqError) as ei:
            tcq.tcq_make_codebook(L, V, 1)
        assert ei.value.status == _lib.TCQ_EINVAL
    assert _lib.load().tcq_make_codebook(4, 1, 0, None) == _lib.TCQ_EINVAL
    assert "NULL" in tcq.tcq_last_error()


def _enc(**kw):
    args = dict(W=FAKE, M=4, N=256, ldw=256, d=None, codebook=FAKE, L=16, k=2, V=1, T=256,
                bitstream=FAKE, start_state=FAKE, cost=FAKE, recon=None, ldr=256,
                workspace=FAKE, workspace_bytes=1, stream=None)
    args.update(kw)
    lib = _lib.load()
    return lib.tcq_encode(args["W"], args["M"], args["N"], args["ldw"], args["d"],
                          args["codebook"], args["L"], args["k"], args["V"], args["T"],
                          args["bitstream"], args["start_state"], args["cost"],
                          args["recon"], args["ldr"], args["workspace"],
                          args["workspace_bytes"], args["stream"])


def test_encode_argument_checks():
    E = _lib
    assert _enc(N=250) == E.TCQ_EINVAL                  # N % T
    assert _enc(T=255, V=2, N=255 * 4) == E.TCQ_EINVAL  # T % V
    assert _enc(k=16, L=16) == E.TCQ_EINVAL             # kV == L
    assert _enc(k=2, V=2, L=4, T=256) == E.TCQ_EINVAL   # kV == L with V > 1
    assert _enc(k=9, L=8) == E.TCQ_EINVAL               # kV > L
    assert _enc(M=-1) == E.TCQ_EINVAL
    assert _enc(L=17) == E.TCQ_EUNSUPPORTED
    assert _enc(k=3, V=3, T=255, N=255, L=16) == E.TCQ_EUNSUPPORTED  # kV = 9 > 8
    assert _enc(V=5, T=260, N=260, L=16, k=1) == E.TCQ_EUNSUPPORTED
    assert _enc(T=2048, N=2048) == E.TCQ_EUNSUPPORTED   # more than 1024 steps
    assert _enc(ldw=100) == E.TCQ_EINVAL
    assert _enc(W=None) == E.TCQ_EINVAL
    assert _enc(codebook=None) == E.TCQ_EINVAL
    assert _enc(bitstream=None) == E.TCQ_EINVAL
    assert _enc(start_state=None) == E.TCQ_EINVAL
    assert _enc(cost=None) == E.TCQ_EINVAL
    assert _enc(recon=FAKE, ldr=3) == E.TCQ_EINVAL
    assert _enc(workspace_bytes=16) == E.TCQ_EWORKSPACE
    assert _enc(workspace=None, workspace_bytes=1 << 40) == E.TCQ_EWORKSPACE
    assert _enc(workspace=FAKE + 4, workspace_bytes=1 << 40) == E.TCQ_EINVAL  # alignment
    assert "256-byte" in tcq.tcq_last_error()
    assert "workspace" in tcq.tcq_last_error()
    # empty problems are a no-op and touch nothing
    assert _enc(M=0) == E.TCQ_OK
    assert _enc(N=0, ldw=0) == E.TCQ_OK
    assert tcq.tcq_last_error() == ""


def test_decode_argument_checks():
    lib = _lib.load()
    E = _lib

    def dec(**kw):
        a = dict(bits=FAKE, s0=FAKE, cb=FAKE, M=2, N=512, L=16, k=2, V=1, T=256, out=FAKE,
                 ldo=512)
        a.update(kw)
        return lib.tcq_decode(a["bits"], a["s0"], a["cb"], a["M"], a["N"], a["L"], a["k"],
                              a["V"], a["T"], a["out"], a["ldo"], None)

    assert dec(N=500) == E.TCQ_EINVAL
    assert dec(bits=None) == E.TCQ_EINVAL
    assert dec(out=None) == E.TCQ_EINVAL
    assert dec(ldo=10) == E.TCQ_EINVAL
    assert dec(L=20) == E.TCQ_EUNSUPPORTED
    assert dec(M=0) == E.TCQ_OK


def test_decode_gemv_argument_checks():
    lib = _lib.load()
    E = _lib

    def gemv(**kw):
        a = dict(bits=FAKE, s0=FAKE, cb=FAKE, M=2, N=512, L=16, k=2, V=1, T=256, x=FAKE,
                 y=FAKE)
        a.update(kw)
        return lib.tcq_decode_gemv(a["bits"], a["s0"], a["cb"], a["M"], a["N"], a["L"],
                                   a["k"], a["V"], a["T"], a["x"], a["y"], None)

    assert gemv(N=500) == E.TCQ_EINVAL
    assert gemv(x=None) == E.TCQ_EINVAL
    assert gemv(y=None) == E.TCQ_EINVAL
    assert gemv(k=16) == E.TCQ_EINVAL
    assert gemv(L=20) == E.TCQ_EUNSUPPORTED
    assert gemv(M=1 << 31) == E.TCQ_EUNSUPPORTED
    assert "exceed" in tcq.tcq_last_error()
    assert gemv(M=0) == E.TCQ_OK


def test_encode_ldlq_argument_checks():
    lib = _lib.load()
    E = _lib

    def run(**kw):
        a = dict(W=FAKE, M=2, N=512, ldw=512, U=FAKE, ldu=512, d=None, cb=FAKE, L=16, k=2,
                 V=1, T=256, bits=FAKE, s0=FAKE, cost=FAKE, recon=None, ldr=512, tgt=None,
                 ldt=512, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.tcq_encode_ldlq(a["W"], a["M"], a["N"], a["ldw"], a["U"], a["ldu"], a["d"],
                                   a["cb"], a["L"], a["k"], a["V"], a["T"], a["bits"],
                                   a["s0"], a["cost"], a["recon"], a["ldr"], a["tgt"],
                                   a["ldt"], a["ws"], a["wsb"], None)

    assert run(N=500) == E.TCQ_EINVAL
    assert run(U=None) == E.TCQ_EINVAL
    assert run(ldu=100) == E.TCQ_EINVAL
    assert run(ldw=100) == E.TCQ_EINVAL
    assert run(recon=FAKE, ldr=10) == E.TCQ_EINVAL
    assert run(tgt=FAKE, ldt=10) == E.TCQ_EINVAL
    assert run(L=20) == E.TCQ_EUNSUPPORTED
    assert run(wsb=100) == E.TCQ_EWORKSPACE
    assert run(ws=FAKE + 4) == E.TCQ_EINVAL                   # not 256-byte aligned
    assert run(M=0) == E.TCQ_OK
    assert tcq.tcq_ldlq_workspace_bytes(0, 512, 16, 2, 1, 256) == 0
    big = tcq.tcq_ldlq_workspace_bytes(4, 512, 16, 2, 1, 256)
    enc = tcq.tcq_encode_workspace_bytes(4, 256, 16, 2, 1, 256)
    assert big >= enc + 4 * 512 * 4 + 4 * 256 * 4


def test_workspace_sizes():
    mn = tcq.tcq_encode_workspace_min_bytes(16, 2, 1, 256)
    full = tcq.tcq_encode_workspace_bytes(2048, 2048, 16, 2, 1, 256)
    assert 0 < mn <= full
    # backpointers alone are n * 2^(L-kV) * kV bits per block
    assert mn >= 256 * (1 << 14) * 2 // 8
    small = tcq.tcq_encode_workspace_bytes(64, 64, 8, 2, 1, 64)
    assert small >= 64 * 64 * 64 * 2 // 8
    with pytest.raises(tcq.TcqError):
        tcq.tcq_encode_workspace_bytes(10, 100, 16, 2, 1, 256)


def test_bcjr_argument_checks():
    lib = _lib.load()
    E = _lib

    def run(**kw):
        a = dict(W=FAKE, M=2, N=512, ldw=512, d=None, cb=FAKE, L=16, k=2, V=1, T=256,
                 tau=0.1, soft=FAKE, ldo=512, logz=None, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.tcq_bcjr(a["W"], a["M"], a["N"], a["ldw"], a["d"], a["cb"], a["L"],
                            a["k"], a["V"], a["T"], a["tau"], a["soft"], a["ldo"], a["logz"],
                            a["ws"], a["wsb"], None)

    assert run(N=500) == E.TCQ_EINVAL                     # N % T
    assert run(k=3, V=2, T=256) == E.TCQ_EUNSUPPORTED     # k*V = 6 > 4
    assert "k*V" in tcq.tcq_last_error()
    assert run(tau=0.0) == E.TCQ_EINVAL
    assert run(tau=-1.0) == E.TCQ_EINVAL
    assert run(tau=float("inf")) == E.TCQ_EINVAL
    assert run(tau=float("nan")) == E.TCQ_EINVAL
    assert run(tau=1e-39) == E.TCQ_EINVAL                  # -log2(e)/tau overflows fp32
    assert run(W=None) == E.TCQ_EINVAL
    assert run(cb=None) == E.TCQ_EINVAL
    assert run(soft=None) == E.TCQ_EINVAL
    assert run(ldw=100) == E.TCQ_EINVAL
    assert run(ldo=100) == E.TCQ_EINVAL
    assert run(wsb=16) == E.TCQ_EWORKSPACE
    assert run(ws=None) == E.TCQ_EWORKSPACE
    assert run(ws=FAKE + 16) == E.TCQ_EINVAL                 # not 256-byte aligned
    assert run(M=0) == E.TCQ_OK
    assert tcq.tcq_last_error() == ""
    size = ctypes_size()
    assert lib.tcq_bcjr_workspace_bytes(2, 512, 16, 2, 1, 256, size) == E.TCQ_OK
    # at least one block: T/V steps of 2^(L-kV) floats (the stored forward vectors)
    assert size.contents.value >= 256 * (1 << 14) * 4
    assert lib.tcq_bcjr_workspace_bytes(2, 512, 16, 4, 2, 256, size) == E.TCQ_EUNSUPPORTED


def test_hadamard_argument_checks():
    lib = _lib.load()
    E = _lib

    def run(**kw):
        a = dict(X=FAKE, rows=2, len=2048, ldx=2048, n=2048, sigma=None, inverse=0,
                 Y=FAKE + (1 << 24), ldy=2048)
        a.update(kw)
        return lib.tcq_hadamard(a["X"], a["rows"], a["len"], a["ldx"], a["n"], a["sigma"],
                                a["inverse"], a["Y"], a["ldy"], None)

    assert run(n=3) == E.TCQ_EINVAL                       # not a power of two
    assert run(n=0) == E.TCQ_EINVAL
    assert run(rows=-1) == E.TCQ_EINVAL
    assert run(len=3000, ldx=3000, ldy=3000) == E.TCQ_EINVAL   # n does not divide len
    assert run(n=8192, len=8192, ldx=8192, ldy=8192) == E.TCQ_EUNSUPPORTED
    assert run(n=32, len=16384, ldx=16384, ldy=16384) == E.TCQ_EUNSUPPORTED
    assert run(X=None) == E.TCQ_EINVAL
    assert run(Y=None) == E.TCQ_EINVAL
    assert run(ldx=1000) == E.TCQ_EINVAL
    assert run(Y=FAKE + 4) == E.TCQ_EINVAL                # overlapping, not the same buffer
    assert "overlap" in tcq.tcq_last_error()
    assert run(Y=FAKE, ldy=4096, ldx=2048) == E.TCQ_EINVAL  # in place needs ldx == ldy
    assert run(rows=0) == E.TCQ_OK
    assert run(len=0, ldx=0, ldy=0) == E.TCQ_OK


def test_scale_field_argument_checks():
    lib = _lib.load()
    E = _lib

    def run(**kw):
        a = dict(W=FAKE, M=4, N=256, ldw=256, a=FAKE, b=FAKE, Wn=None, ldn=256, ws=FAKE,
                 wsb=1 << 40)
        a.update(kw)
        return lib.tcq_scale_field(a["W"], a["M"], a["N"], a["ldw"], a["a"], a["b"], a["Wn"],
                                   a["ldn"], a["ws"], a["wsb"], None)

    assert run(M=-1) == E.TCQ_EINVAL
    assert run(W=None) == E.TCQ_EINVAL
    assert run(a=None) == E.TCQ_EINVAL
    assert run(b=None) == E.TCQ_EINVAL
    assert run(ldw=100) == E.TCQ_EINVAL
    assert run(Wn=FAKE, ldn=100) == E.TCQ_EINVAL
    assert run(wsb=16) == E.TCQ_EWORKSPACE
    assert run(ws=None) == E.TCQ_EWORKSPACE
    assert run(ws=FAKE + 8) == E.TCQ_EINVAL                  # not 256-byte aligned
    assert run(M=0) == E.TCQ_OK
    assert run(N=0) == E.TCQ_OK
    size = ctypes_size()
    assert lib.tcq_scale_field_workspace_bytes(4, 256, size) == E.TCQ_OK
    assert size.contents.value == 4 * 256 * 4                 # one slab per row when M < 64
    assert lib.tcq_scale_field_workspace_bytes(4096, 256, size) == E.TCQ_OK
    assert size.contents.value == 64 * 256 * 4                # 64 slabs of column sums


def ctypes_size():
    import ctypes
    return ctypes.pointer(ctypes.c_size_t(0))


def test_stream_probe_argument_checks():
    lib = _lib.load()
    E = _lib
    assert lib.tcq_l16_stream_probe_bytes(0) == 0
    assert lib.tcq_l16_stream_probe_bytes(2) == 3 * 65536 * 4 + 2 * 512 * 4
    need = lib.tcq_l16_stream_probe_bytes(4)
    assert lib.tcq_l16_stream_probe(0, 1, FAKE, need, None, None, None) == E.TCQ_EINVAL
    assert lib.tcq_l16_stream_probe(4, 0, FAKE, need, None, None, None) == E.TCQ_EINVAL
    assert lib.tcq_l16_stream_probe(4, 1, None, need, None, None, None) == E.TCQ_EINVAL
    assert lib.tcq_l16_stream_probe(4, 1, FAKE, need - 1, None, None, None) == E.TCQ_EINVAL
    assert lib.tcq_l16_stream_probe(4, 1, FAKE + 8, need, None, None, None) == E.TCQ_EINVAL

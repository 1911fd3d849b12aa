"""ctypes binding of libtcq.so (include/tcq.h): same names, argument marshalling only.

Device buffers are passed as integer addresses (for torch tensors: ``t.data_ptr()``),
streams as integer ``hipStream_t`` handles (``torch.cuda.current_stream().cuda_stream``).
There is no fallback: if libtcq.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtcq.so")

TCQ_OK = 0
TCQ_EINVAL = -1
TCQ_EUNSUPPORTED = -2
TCQ_EWORKSPACE = -3
TCQ_EHIP = -4
TCQ_ENOMEM = -5

EXPORTED = ("tcq_version", "tcq_last_error", "tcq_make_codebook",
            "tcq_encode_workspace_bytes", "tcq_encode_workspace_min_bytes", "tcq_encode",
            "tcq_encode_timed", "tcq_encode_noalloc", "tcq_decode", "tcq_decode_gemv",
            "tcq_ldlq_workspace_bytes", "tcq_encode_ldlq", "tcq_bcjr_workspace_bytes",
            "tcq_bcjr", "tcq_hadamard", "tcq_scale_field_workspace_bytes", "tcq_scale_field",
            "tcq_l16_stream_probe_bytes", "tcq_l16_stream_probe")

_lib = None


class TcqError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtcq.so not found at {LIB_PATH}; build it with "
                          "trellis_coded_bit_amd/build.py (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.tcq_version.restype = i32
    lib.tcq_version.argtypes = []
    lib.tcq_last_error.restype = ctypes.c_char_p
    lib.tcq_last_error.argtypes = []
    lib.tcq_make_codebook.restype = i32
    lib.tcq_make_codebook.argtypes = [i32, i32, ctypes.c_uint64, vp]
    lib.tcq_encode_workspace_bytes.restype = i32
    lib.tcq_encode_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32,
                                               ctypes.POINTER(sz)]
    lib.tcq_encode_workspace_min_bytes.restype = i32
    lib.tcq_encode_workspace_min_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.tcq_encode.restype = i32
    lib.tcq_encode.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp,
                               i64, vp, sz, vp]
    lib.tcq_encode_timed.restype = i32
    lib.tcq_encode_timed.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, vp, vp, vp,
                                     vp, i64, vp, sz, vp, vp, vp]
    lib.tcq_encode_noalloc.restype = i32
    lib.tcq_encode_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, vp, vp,
                                       vp, vp, i64, vp]
    lib.tcq_decode.restype = i32
    lib.tcq_decode.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, vp, i64, vp]
    lib.tcq_l16_stream_probe_bytes.restype = sz
    lib.tcq_l16_stream_probe_bytes.argtypes = [i64]
    lib.tcq_l16_stream_probe.restype = i32
    lib.tcq_l16_stream_probe.argtypes = [i64, i32, vp, sz, vp, vp, vp]
    lib.tcq_decode_gemv.restype = i32
    lib.tcq_decode_gemv.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, vp, vp, vp]
    lib.tcq_ldlq_workspace_bytes.restype = i32
    lib.tcq_ldlq_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.tcq_encode_ldlq.restype = i32
    lib.tcq_encode_ldlq.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, i32, i32, i32, i32,
                                    vp, vp, vp, vp, i64, vp, i64, vp, sz, vp]
    lib.tcq_bcjr_workspace_bytes.restype = i32
    lib.tcq_bcjr_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.tcq_bcjr.restype = i32
    lib.tcq_bcjr.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                             vp, i64, vp, vp, sz, vp]
    lib.tcq_hadamard.restype = i32
    lib.tcq_hadamard.argtypes = [vp, i64, i64, i64, i64, vp, i32, vp, i64, vp]
    lib.tcq_scale_field_workspace_bytes.restype = i32
    lib.tcq_scale_field_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.tcq_scale_field.restype = i32
    lib.tcq_scale_field.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, vp, sz, vp]
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != TCQ_OK:
        raise TcqError(fn, rc, load().tcq_last_error().decode())


def tcq_version() -> int:
    return load().tcq_version()


def tcq_last_error() -> str:
    return load().tcq_last_error().decode()


def tcq_make_codebook(L: int, V: int, seed: int) -> np.ndarray:
    out = np.empty((1 << L, V), dtype=np.float32)
    _check("tcq_make_codebook",
           load().tcq_make_codebook(L, V, seed & 0xFFFFFFFFFFFFFFFF, out.ctypes.data))
    return out


def tcq_encode_workspace_bytes(M: int, N: int, L: int, k: int, V: int, T: int) -> int:
    b = ctypes.c_size_t(0)
    _check("tcq_encode_workspace_bytes",
           load().tcq_encode_workspace_bytes(M, N, L, k, V, T, ctypes.byref(b)))
    return int(b.value)


def tcq_encode_workspace_min_bytes(L: int, k: int, V: int, T: int) -> int:
    b = ctypes.c_size_t(0)
    _check("tcq_encode_workspace_min_bytes",
           load().tcq_encode_workspace_min_bytes(L, k, V, T, ctypes.byref(b)))
    return int(b.value)


def tcq_encode(W: int, M: int, N: int, ldw: int, d: int | None, codebook: int, L: int,
               k: int, V: int, T: int, bitstream: int, start_state: int, cost: int,
               recon: int | None, ldr: int, workspace: int, workspace_bytes: int,
               stream: int | None) -> None:
    _check("tcq_encode",
           load().tcq_encode(W, M, N, ldw, d or None, codebook, L, k, V, T, bitstream,
                             start_state, cost, recon or None, ldr, workspace,
                             workspace_bytes, stream or None))


def tcq_encode_timed(W: int, M: int, N: int, ldw: int, d: int | None, codebook: int, L: int,
                     k: int, V: int, T: int, bitstream: int, start_state: int, cost: int,
                     recon: int | None, ldr: int, workspace: int, workspace_bytes: int,
                     stream: int | None, acs_begin: int | None, acs_end: int | None) -> None:
    _check("tcq_encode_timed",
           load().tcq_encode_timed(W, M, N, ldw, d or None, codebook, L, k, V, T, bitstream,
                                   start_state, cost, recon or None, ldr, workspace,
                                   workspace_bytes, stream or None, acs_begin or None,
                                   acs_end or None))


def tcq_encode_noalloc(W: int, M: int, N: int, ldw: int, d: int | None, codebook: int,
                       L: int, k: int, V: int, T: int, bitstream: int, start_state: int,
                       cost: int, recon: int | None, ldr: int, stream: int | None) -> None:
    _check("tcq_encode_noalloc",
           load().tcq_encode_noalloc(W, M, N, ldw, d or None, codebook, L, k, V, T, bitstream,
                                     start_state, cost, recon or None, ldr, stream or None))


def tcq_l16_stream_probe_bytes(blocks: int) -> int:
    return int(load().tcq_l16_stream_probe_bytes(blocks))


def tcq_l16_stream_probe(blocks: int, super_steps: int, workspace: int, workspace_bytes: int,
                         stream: int | None, start: int | None, stop: int | None) -> None:
    _check("tcq_l16_stream_probe",
           load().tcq_l16_stream_probe(blocks, super_steps, workspace, workspace_bytes,
                                       stream or None, start or None, stop or None))


def tcq_decode(bitstream: int, start_state: int, codebook: int, M: int, N: int, L: int,
               k: int, V: int, T: int, out: int, ldo: int, stream: int | None) -> None:
    _check("tcq_decode",
           load().tcq_decode(bitstream, start_state, codebook, M, N, L, k, V, T, out, ldo,
                             stream or None))


def tcq_decode_gemv(bitstream: int, start_state: int, codebook: int, M: int, N: int, L: int,
                    k: int, V: int, T: int, x: int, y: int, stream: int | None) -> None:
    _check("tcq_decode_gemv",
           load().tcq_decode_gemv(bitstream, start_state, codebook, M, N, L, k, V, T, x, y,
                                  stream or None))


def tcq_ldlq_workspace_bytes(M: int, N: int, L: int, k: int, V: int, T: int) -> int:
    b = ctypes.c_size_t(0)
    _check("tcq_ldlq_workspace_bytes",
           load().tcq_ldlq_workspace_bytes(M, N, L, k, V, T, ctypes.byref(b)))
    return int(b.value)


def tcq_encode_ldlq(W: int, M: int, N: int, ldw: int, U: int | None, ldu: int,
                    d: int | None, codebook: int, L: int, k: int, V: int, T: int,
                    bitstream: int, start_state: int, cost: int, recon: int | None, ldr: int,
                    target: int | None, ldt: int, workspace: int, workspace_bytes: int,
                    stream: int | None) -> None:
    _check("tcq_encode_ldlq",
           load().tcq_encode_ldlq(W, M, N, ldw, U or None, ldu, d or None, codebook, L, k, V,
                                  T, bitstream, start_state, cost, recon or None, ldr,
                                  target or None, ldt, workspace, workspace_bytes,
                                  stream or None))


def tcq_bcjr_workspace_bytes(M: int, N: int, L: int, k: int, V: int, T: int) -> int:
    b = ctypes.c_size_t(0)
    _check("tcq_bcjr_workspace_bytes",
           load().tcq_bcjr_workspace_bytes(M, N, L, k, V, T, ctypes.byref(b)))
    return int(b.value)


def tcq_bcjr(W: int, M: int, N: int, ldw: int, d: int | None, codebook: int, L: int, k: int,
             V: int, T: int, tau: float, soft: int, ldo: int, logz: int | None, workspace: int,
             workspace_bytes: int, stream: int | None) -> None:
    _check("tcq_bcjr",
           load().tcq_bcjr(W, M, N, ldw, d or None, codebook, L, k, V, T, tau, soft, ldo,
                           logz or None, workspace, workspace_bytes, stream or None))


def tcq_hadamard(X: int, rows: int, length: int, ldx: int, n: int, sigma: int | None,
                 inverse: bool, Y: int, ldy: int, stream: int | None) -> None:
    _check("tcq_hadamard",
           load().tcq_hadamard(X, rows, length, ldx, n, sigma or None, 1 if inverse else 0, Y,
                               ldy, stream or None))


def tcq_scale_field_workspace_bytes(M: int, N: int) -> int:
    b = ctypes.c_size_t(0)
    _check("tcq_scale_field_workspace_bytes",
           load().tcq_scale_field_workspace_bytes(M, N, ctypes.byref(b)))
    return int(b.value)


def tcq_scale_field(W: int, M: int, N: int, ldw: int, row_scale: int, col_scale: int,
                    Wn: int | None, ldn: int, workspace: int, workspace_bytes: int,
                    stream: int | None) -> None:
    _check("tcq_scale_field",
           load().tcq_scale_field(W, M, N, ldw, row_scale, col_scale, Wn or None, ldn,
                                  workspace, workspace_bytes, stream or None))

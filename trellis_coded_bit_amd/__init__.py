"""trellis_coded_bit_amd: bitshift-trellis Viterbi encoder on AMD MI355X.

The compute lives in libtcq.so (HIP kernels for gfx950 behind the C ABI in
include/tcq.h).  ``_lib`` mirrors that ABI with ctypes; ``api`` adds torch-allocated
buffers and streams; ``workloads`` makes seeded synthetic inputs.
"""
from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    TcqError,
    tcq_decode,
    tcq_decode_gemv,
    tcq_ldlq_workspace_bytes,
    tcq_encode_ldlq,
    tcq_bcjr_workspace_bytes,
    tcq_bcjr,
    tcq_hadamard,
    tcq_scale_field_workspace_bytes,
    tcq_scale_field,
    tcq_encode,
    tcq_encode_timed,
    tcq_encode_workspace_bytes,
    tcq_encode_workspace_min_bytes,
    tcq_last_error,
    tcq_make_codebook,
    tcq_version,
)

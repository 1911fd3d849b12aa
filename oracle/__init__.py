"""CPU oracle for the bitshift-trellis Viterbi encoder (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of bench.py may import
this package.  The GPU library never links or calls it.
"""
from .oracle import (  # noqa: F401
    build,
    lib_path,
    inv_normal_cdf,
    splitmix64_stream,
    make_codebook,
    encode_block,
    two_best_block,
    decode_block,
    path_cost,
    encode_matrix,
    nwords,
    decode_matrix,
    decode_gemv,
    ldlq_encode,
    bcjr_block,
    bcjr_matrix,
    hadamard,
    scale_field,
)

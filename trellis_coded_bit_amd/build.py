"""Build libtcq.so in-tree with hipcc for gfx950.

Every source is compiled to its own object (in parallel), then the objects are linked
into the shared library.  Objects live in trellis_coded_bit_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtcq.so")
OBJDIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["tcq_api.cpp", "codebook.cpp", "kernels_generic.hip", "kernels_l16.hip",
           "kernels_l16k3.hip", "kernels_l16h.hip", "kernels_ldlq.hip", "kernels_bcjr.hip",
           "kernels_preprocess.hip", "kernels_decode.hip", "tcq_noalloc.hip"]

# -ffp-contract=off: the encoder's fp32 recurrence is written with explicit fmaf and
#   must not gain extra contractions.
# -fno-gpu-flush-denormals-to-zero: keep IEEE denormals on the device.
# -packed-fp32-ops removed from the target features: no v_pk_*_f32 is generated.
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# The target feature above is meant for the gfx950 device pass.  clang hands -Xclang
# options to the x86 host pass as well (-Xarch_device refuses options that take an
# argument), and the host pass prints this line for it and ignores the feature.  Only
# that exact line is dropped from the compiler output; every other diagnostic is shown.
_HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _filter(text: str) -> str:
    return "".join(line for line in text.splitlines(keepends=True)
                   if _HOST_FEATURE_NOTE not in line)


def _compile(src: str) -> tuple[str, subprocess.CompletedProcess]:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj,
           os.path.join(CSRC, src)]
    return obj, subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(_compile, SOURCES))
    failed = False
    for obj, res in results:
        msg = _filter(res.stdout + res.stderr)
        if msg.strip():
            sys.stderr.write(msg)
        if res.returncode != 0:
            failed = True
    if failed:
        raise RuntimeError("hipcc failed to build libtcq.so")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[obj for obj, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = _filter(res.stdout + res.stderr)
    if msg.strip():
        sys.stderr.write(msg)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed to link libtcq.so")
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"built {LIB} from {len(SOURCES)} sources\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

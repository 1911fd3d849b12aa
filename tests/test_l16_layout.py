"""Host check of the L = 16 kernel's index math (slot <-> state bijections, group
structure, the three-step transposition, LDS staging addresses and bank spread, the
transposition rounds spread over the segments, and the k*V = 4 segment-pair order).
Compiles tests/l16_layout_check.cpp against the kernel's own layout header with g++
and runs it on the CPU."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_l16_layout(tmp_path):
    exe = tmp_path / "l16chk"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I",
                    os.path.join(ROOT, "trellis_coded_bit_amd", "csrc"),
                    os.path.join(ROOT, "tests", "l16_layout_check.cpp"), "-o", str(exe)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "l16 layout ok" in res.stdout

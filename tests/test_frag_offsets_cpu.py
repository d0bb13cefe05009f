"""The kernels' LDS fragment offsets (FragOffsets in csrc/common.h, a lane
base XOR a constant) equal the swizzled tile layout's element-wise offsets
for every lane and fragment. Compiles a host-only check against the real
header; no GPU needed."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_frag_offsets_match_tile_layout(tmp_path):
    exe = tmp_path / "frag_offsets_check"
    src = os.path.join(ROOT, "tests", "frag_offsets_check.cpp")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "ulysses_sequence_parallelism_seq_amd", "csrc"),
                    src, "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches d=64: 0 d=128: 0" in r.stdout
    assert "natural-order transposing reads, mismatches d=64: 0 d=128: 0" in r.stdout

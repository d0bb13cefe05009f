"""The persistent launches' tile lists (queue_decode in csrc/common.h) hand
out every tile exactly once, each XCD's list only its own units, in level
groups and unit by unit. Compiles a host-only check against the real header;
no GPU needed."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_tile_queue_lists_cover_every_tile_once(tmp_path):
    exe = tmp_path / "tile_queue_check"
    src = os.path.join(ROOT, "tests", "tile_queue_check.cpp")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "ulysses_sequence_parallelism_seq_amd", "csrc"),
                    src, "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout

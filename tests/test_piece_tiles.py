"""Host check of the per-sample query-tile map the bf16 walk and the dQ pass
use (positions.h: fill_piece_tiles, piece_tile).  A C++ program built with
g++ against the HIP headers runs the map over 600 seeded random packings of
1..256 samples and checks that every row of the share lies in exactly one
tile, inside one piece (one sample's chunk r or 2cp - 1 - r), within the
tile's row limit.  No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_ring_attention_amd", "csrc")
HIP_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INC), reason="g++ or HIP headers missing")
def test_piece_tile_map_covers_every_row_once(tmp_path):
    exe = str(tmp_path / "piece_tiles_check")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", HIP_INC, "-I", CSRC, os.path.join(ROOT, "tests", "c", "piece_tiles_check.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "piece tiles ok 600"

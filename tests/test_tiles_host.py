"""Host logic of the band-tile scheduler: the multiply-based divisions and the
division-free tile decoder the persistent kernels use, checked against plain integer
division by a small g++ program (tests/host/tiles_check.cpp)."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "sliding_window_attention_diagmm_amd", "csrc")


def test_tile_decoder_matches_division():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "tiles_check")
        build = subprocess.run(
            ["g++", "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "host", "tiles_check.cpp"),
             "-o", exe], capture_output=True, text=True)
        if build.returncode != 0:
            pytest.fail("g++ failed:\n" + build.stderr[-2000:])
        run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr

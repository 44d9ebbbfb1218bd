"""The MFMA kernels' tile decode on the host: tests/decode_check.hip includes
the kernel headers and calls the same decode functions the kernels run
(decode_tile_at, decode_half_tile, split_first_half), compiled for the host
only, and checks that every launch layout covers each output block exactly
once (plain grid, expert segments with padding rows, the grouped forward's
split launch, expert-local reductions).  No GPU is involved."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_tile_decode_covers_every_block_once(tmp_path):
    exe = tmp_path / "decode_check"
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "deterministic_invariant_gemm_amd", "csrc"),
           os.path.join(HERE, "decode_check.hip"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "decode ok" in r.stdout
    # the config-5-like shapes take both launch layouts
    assert "16384 n=1408 e=8: 576 slots, split" in r.stdout
    assert "20000 n=1408 e=16: 576 slots, whole slots" in r.stdout

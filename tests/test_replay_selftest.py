"""The launch replay checks itself: replay_selftest.cpp drives the host-side
replay of the block-update and trailing-update kernels with hand-built
launches.  Buffers registered to cover every access exactly must pass, and a
buffer registered one element short (the last 16-byte vector load of an
operand then crosses its end), a misaligned vector operand and an output
registered read-only must each be rejected, with the access named.  CPU
only: the program is built with hipcc and makes no HIP call."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_replay_rejects_planted_out_of_bounds_accesses(tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    exe = tmp_path / "replay_selftest"
    cmd = [HIPCC, "-std=c++17", "-O1", "--offload-arch=gfx950", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "cholesky_spd_solve_amd", "csrc"), os.path.join(HERE, "replay_selftest.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert sum(line.startswith("ok: ") for line in lines) == 6
    assert "reads 16 bytes" in r.stdout and "unaligned vector load" in r.stdout

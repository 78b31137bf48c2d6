"""The balanced schedule's unit arithmetic (csrc/common.h: sched_real,
sched_virtual, unit_begin, g_of_unit), built for the host from the same
header the kernels use and checked exhaustively on seeded random launches by
tests/sched_check.cpp: consistent virtual <-> real maps, no empty workgroup
range, and every unit owned by the workgroup that covers it (the split merge
finds a query tile's partial states through that ownership)."""
import os
import shutil
import subprocess

import pytest

from kv_cache_attention_chunk_amd import build as pkg

HERE = os.path.dirname(os.path.abspath(__file__))


def test_schedule_arithmetic(tmp_path):
    hipcc = pkg.hipcc()
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "sched_check"
    cmd = [hipcc, "--offload-host-only", "-O2", "-std=c++17", "-I", pkg.CSRC,
           os.path.join(HERE, "sched_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

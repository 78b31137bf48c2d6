"""The C ABI from a caller with no Python and no torch: tests/c_abi_driver.cpp
(built by __graft_entry__.build() into tests/_bin/) allocates its own device
buffers, runs dense chunk attention and the same attention as two key ranges
recombined by the LSE merge, checks that a bad head dim is rejected, and
writes the outputs; they are compared here with the CPU oracle on the whole
output (O max-abs 1e-2 plus the bf16 output half-ulp from |O| = 2, LSE
max-abs 1e-3).  The driver's inputs come from a counter formula that this
test reproduces."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as orc
from helpers import assert_lse, assert_o

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "_bin", "c_abi_driver")
B, H, NQ, NKV, D = 1, 2, 200, 500, 128


def _gen(n, s):
    """Element i of tensor s: ((hash(i + s 2^24) >> 13) & 255) - 128, over
    128, with hash(x) = x * 2654435761 mod 2^32 (the driver's formula)."""
    i = np.arange(n, dtype=np.uint64) + np.uint64(s << 24)
    x = (i * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    return (((x >> np.uint64(13)) & np.uint64(255)).astype(np.float64) - 128.0) / 128.0


def _bf16_file(path, shape):
    bits = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64).reshape(shape)


def test_c_abi_driver(tmp_path):
    print("[gpu-case] C ABI driver: dense and split + LSE merge, B=1 H=2 Nq=200 Nkv=500 d=128",
          flush=True)
    sys.stdout.flush()
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build()"
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"driver failed ({r.returncode}): {r.stderr}"
    Q = _gen(B * NQ * H * D, 0).reshape(B, NQ, H, D)
    K = _gen(B * NKV * H * D, 1).reshape(B, NKV, H, D)
    V = _gen(B * NKV * H * D, 2).reshape(B, NKV, H, D)
    Or, Lr = orc.chunk_attn_dense(Q, K, V, 1 / math.sqrt(D))
    o = _bf16_file(tmp_path / "o_dense.bf16", (B, NQ, H, D))
    lse = np.fromfile(tmp_path / "lse_dense.f32", dtype=np.float32).reshape(B, H, NQ)
    assert_o(o, Or, True, "C driver dense")
    assert_lse(lse, Lr, "C driver dense")
    om = _bf16_file(tmp_path / "o_merged.bf16", (B, NQ, H, D))
    lm = np.fromfile(tmp_path / "lse_merged.f32", dtype=np.float32).reshape(B, H, NQ)
    assert_o(om, Or, True, "C driver split + merge")
    assert_lse(lm, Lr, "C driver split + merge")

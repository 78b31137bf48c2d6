"""GPU parity of ragged cache packing (Pyramid Forcing page, sections 2-3):
per-head frame copies and adjacent-frame merges flattened into K/V buffers
with cu_seqlens, bit-exact against the CPU oracle; attention over the
GPU-packed caches checked against the oracle on its own packed caches."""
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
import oracle as orc
from kv_cache_attention_chunk_amd import workloads as wl
from helpers import assert_lse, assert_o, i32, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _src(frames):
    ptr = np.zeros(len(frames) + 1, np.int64)
    src = []
    for bh, fl in enumerate(frames):
        for f in fl:
            src.append(tuple(f) if isinstance(f, tuple) else (f, -1))
        ptr[bh + 1] = len(src)
    return ptr, np.array(src, np.int64).reshape(-1, 2)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d", [64, 128])
def test_pack_small_copies_merges_and_edges(d):
    say(f"pack small d={d}")
    rng = np.random.default_rng(d)
    B, H, T, nf = 2, 3, 40, 8
    K = wl.Bf16Tensor.from_f32(rng.standard_normal((B, nf * T + 7, H, d), dtype=np.float32) * 3)
    V = wl.Bf16Tensor.from_f32(rng.standard_normal((B, nf * T + 7, H, d), dtype=np.float32))
    frames = [[0, (2, 3), 7], [], [(1, 1), 5, (6, 7), 9], [4], [(0, 7), (3, 4), 2, 1], [(8, 2)]]
    kf, vf, cu, cu_h = ca.pack_ragged(to_dev(K), to_dev(V), frames, T)
    torch.cuda.synchronize()
    ptr, src = _src(frames)
    rk, rv, rcu = orc.pack_ragged(K.bits, V.bits, ptr, src, T)
    assert np.array_equal(_bits(kf), rk) and np.array_equal(_bits(vf), rv)
    assert np.array_equal(cu.cpu().numpy(), rcu) and np.array_equal(cu_h, rcu)


def test_pack_no_frames():
    say("pack with no frames")
    k = torch.zeros((1, 80, 2, 64), dtype=torch.bfloat16, device="cuda")
    kf, vf, cu, _ = ca.pack_ragged(k, k, [[], []], 40)
    torch.cuda.synchronize()
    assert kf.shape[0] == 0 and cu.cpu().tolist() == [0, 0, 0]


def test_pack_ragged_workload_and_attention():
    say("pack the 12-head ragged workload, then ragged attention on it")
    w = wl.ragged(seed=0)
    frames = [w.ragged_frames[bh] for bh in range(w.B * w.H)]
    k, v = to_dev(w.k), to_dev(w.v)
    kf, vf, cu, cu_h = ca.pack_ragged(k, v, frames, 1560)
    torch.cuda.synchronize()
    # the generator's own flattening of the same frame lists (copies only)
    assert np.array_equal(_bits(kf), w.k_flat.bits) and np.array_equal(_bits(vf), w.v_flat.bits)
    assert np.array_equal(cu.cpu().numpy(), w.cu_seqlens)
    o, l = ca.chunk_attn_varlen_fwd(to_dev(w.q), kf, vf, cu, cu_seqlens_host=cu_h, scale=w.scale)
    torch.cuda.synchronize()
    rows = np.r_[0:24, 4660:4680]
    Or, Lr = orc.chunk_attn_varlen(w.q.f32, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens, w.scale, rows=rows)
    assert_o(o[:, rows], Or, True, "packed ragged")
    assert_lse(l[:, :, rows], Lr, "packed ragged")


def test_pack_merged_frames_full_size():
    say("pack with adjacent-frame merges at the Wan shape")
    w = wl.wan_dense(seed=1, head_scales=False)
    k, v = to_dev(w.k), to_dev(w.v)
    # every head: sink, middle frames merged in pairs (a cache-merge policy), recent frames
    frames = []
    for h in range(w.H):
        lo = 1 + (h % 3)
        frames.append([0] + [(f, f + 1) for f in range(lo, 18, 2)] + [18, 19, 20])
    kf, vf, cu, cu_h = ca.pack_ragged(k, v, frames, 1560)
    torch.cuda.synchronize()
    ptr, src = _src(frames)
    rk, rv, rcu = orc.pack_ragged(w.k.bits, w.v.bits, ptr, src, 1560)
    assert np.array_equal(_bits(kf), rk) and np.array_equal(_bits(vf), rv)
    assert np.array_equal(cu.cpu().numpy(), rcu)

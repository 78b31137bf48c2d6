"""Seeded input generators: shapes, determinism, bf16 rounding, ragged layout."""
import numpy as np
import pytest
import torch

from kv_cache_attention_chunk_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-6, 6, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38], np.float32)])
    bits = wl.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = wl.bf16_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_dense_shapes_and_blocks():
    w = wl.tiny_dense(seed=0)
    assert w.q.shape == (1, 256, 2, 64) and w.k.shape == (1, 1024, 2, 64)
    assert w.meta["local_blocks"] == [0, 12, 13, 14, 15]
    assert w.meta["history_blocks"] == list(range(1, 12))
    w2 = wl.tiny_dense(seed=0)
    np.testing.assert_array_equal(w.q.bits, w2.q.bits)
    w3 = wl.tiny_dense(seed=1)
    assert not np.array_equal(w.q.bits, w3.q.bits)
    assert abs(w.k.f32.std() - 1.0) < 0.02


def test_wan_dense_small_frames_layout():
    w = wl.wan_dense(seed=0, H=3, d=16, frames_q=3, frames_kv=21, frame_tokens=100)
    assert w.Nq == 300 and w.Nkv == 2100
    bpf = 2  # 64 + 36
    assert w.meta["blocks_per_frame"] == bpf
    assert w.meta["local_blocks"] == [0, 1] + list(range(36, 42))
    assert w.meta["history_blocks"] == list(range(2, 36))
    s = w.head_scale
    assert s.shape == (3,) and np.all((s >= 0.5) & (s <= 2.0))
    # per-head scale multiplies Q and K, not V
    for h in range(3):
        assert abs(w.k.f32[0, :, h].std() / s[h] - 1.0) < 0.05
        assert abs(w.v.f32[0, :, h].std() - 1.0) < 0.05


@pytest.mark.parametrize("cls", [0, 1, 2])
def test_ragged_frame_subsets(cls):
    for n in range(3, 22):
        fr = wl.ragged_frame_subset(cls, n)
        assert len(fr) == n and len(set(fr)) == n and fr == sorted(fr)
        assert fr[0] == 0 and fr[-2:] == [19, 20]
        assert all(1 <= f <= 18 for f in fr[1:-2])
    assert wl.ragged_frame_subset(2, 6)[1:-2] == [16, 17, 18]
    assert wl.ragged_frame_subset(1, 6)[1:-2] == [6, 12, 18]
    assert wl.ragged_frame_subset(0, 6)[1:-2] == [1, 10, 18]


def test_ragged_layout_small():
    w = wl.ragged(seed=2, H=4, d=8, frames_q=1, frames_kv=6, frame_tokens=20)
    cu = w.cu_seqlens
    assert cu.dtype == np.int32 and cu[0] == 0 and np.all(np.diff(cu) > 0)
    for h in range(4):
        fr = w.ragged_frames[h]
        lo, hi = cu[h], cu[h + 1]
        assert hi - lo == 20 * len(fr)
        got = w.k_flat.bits[lo:hi]
        want = np.concatenate([w.k.bits[0, 20 * f:20 * f + 20, h] for f in fr])
        np.testing.assert_array_equal(got, want)


def test_ragged_full_size_lengths():
    # lengths only; no tensors needed
    rng = np.random.default_rng(0)
    rng.standard_normal((1, 4680, 12, 128), dtype=np.float32)
    w = wl.ragged(seed=0, H=12, d=8)
    L = np.diff(w.cu_seqlens)
    assert np.all(L % 1560 == 0) and L.min() >= 4680 and L.max() <= 32760


def test_mixed_modes_small():
    w = wl.mixed(seed=0, H=6, d=8, frames_q=3, frames_kv=21, frame_tokens=20)
    assert w.head_mode.tolist() == [0, 1, 2, 0, 1, 2]
    L = np.diff(w.cu_seqlens)
    assert L[0] == 0 and L[1] == 0 and L[2] > 0 and L[5] > 0
    lay = w.meta["sparse"]
    assert lay["K"] == int(np.ceil(0.125 * lay["local_count"]))


def test_random_csr_sorted_unique():
    rng = np.random.default_rng(1)
    ip, ix = wl.random_csr(rng, 50, 30, 12)
    assert ip[0] == 0 and ip[-1] == len(ix)
    for r in range(50):
        row = ix[ip[r]:ip[r + 1]]
        assert np.all(np.diff(row) > 0) and (len(row) == 0 or (row.min() >= 0 and row.max() < 30))

"""GPU parity of the balanced schedule: dense and ragged launches whose key
ranges are split over the device's resident workgroups and finished by the
LSE merge of float32 partials, against the CPU oracle.

Shapes are chosen so that the schedule is taken (a head reaches 64 key tiles
and the plain grid would be unbalanced), so that query tiles are cut into
many parts, mid-tile and at ragged key tails, and so that empty heads and
ragged query tails occur.  A workspace pre-filled with NaN shows that the
split path ran: partials overwrite part of it.
"""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
import oracle as orc
from kv_cache_attention_chunk_amd import workloads as wl
from helpers import assert_lse, assert_o, assert_written, i32, nan_lse, nan_out, to_dev, wave_rows

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _gen(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * scale)


def _nan_ws(d):
    n = ca.workspace_bytes(d)
    assert n > 0
    return torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)


def _touched(ws):
    return bool((~torch.isnan(ws.view(torch.float32))).any())


@pytest.mark.parametrize("B,H,Nq,Nkv,d,out_dtype", [
    (1, 3, 300, 4497, 128, torch.bfloat16),      # 71 key tiles, last one 17 keys
    (2, 2, 130, 8197, 64, torch.float32),        # 2 query tiles, the second of 2 rows
    (1, 1, 1, 6000, 128, torch.float32),         # one query row, one tile split many ways
])
def test_balanced_dense(B, H, Nq, Nkv, d, out_dtype):
    say(f"balanced dense B={B} H={H} Nq={Nq} Nkv={Nkv} d={d}")
    Q, K, V = _gen(1, (B, Nq, H, d), 1.3), _gen(2, (B, Nkv, H, d), 1.3), _gen(3, (B, Nkv, H, d))
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    ws = _nan_ws(d)
    o, l = ca.chunk_attn_fwd(q, k, v, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    assert _touched(ws), "balanced schedule not taken"
    Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, 1 / math.sqrt(d))
    assert_o(o, Or, out_dtype == torch.bfloat16, "balanced dense")
    assert_lse(l, Lr, "balanced dense")
    # the plain grid gives the same attention
    o2, l2 = ca.chunk_attn_fwd(q, k, v, out_dtype=out_dtype, balanced=False)
    torch.cuda.synchronize()
    assert_o(o2, Or, out_dtype == torch.bfloat16, "plain dense")
    assert float((l - l2).abs().max()) < 1e-4


def test_balanced_ragged_with_empty_and_short_heads():
    say("balanced ragged")
    H, Nq, d = 5, 200, 128
    lens = np.array([0, 4100, 130, 2000, 64])
    cu = np.zeros(H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    Q = _gen(4, (1, Nq, H, d))
    Kf, Vf = _gen(5, (int(cu[-1]), d)), _gen(6, (int(cu[-1]), d))
    ws = _nan_ws(d)
    o, l = ca.chunk_attn_varlen_fwd(to_dev(Q), to_dev(Kf), to_dev(Vf), i32(cu),
                                    cu_seqlens_host=cu, workspace=ws)
    torch.cuda.synchronize()
    assert _touched(ws), "balanced schedule not taken"
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, 1 / math.sqrt(d))
    assert_o(o, Or, True, "balanced ragged")
    assert_lse(l, Lr, "balanced ragged")
    assert torch.all(l[:, 0] == -math.inf) and torch.all(o[:, :, 0] == 0)


def test_balanced_mixed_dense_ragged_blocks():
    say("balanced mixed")
    H, Nq, Nkv, d = 6, 260, 4200, 64
    mode = np.array([0, 2, 1, 2, 0, 1], np.int32)
    Q, K, V = _gen(7, (1, Nq, H, d)), _gen(8, (1, Nkv, H, d)), _gen(9, (1, Nkv, H, d))
    lens = np.zeros(H, np.int64)
    lens[1], lens[3] = 5000, 777
    cu = np.zeros(H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    Kf, Vf = _gen(10, (int(cu[-1]), d)), _gen(11, (int(cu[-1]), d))
    seg, blk = 600, 64
    nkb = orc.block_spans(Nkv, blk, seg).shape[0]
    nqb = orc.block_spans(Nq, blk, seg).shape[0]
    rng = np.random.default_rng(12)
    indptr, indices = wl.random_csr(rng, H * nqb, nkb, 20)
    ws = _nan_ws(d)
    o, l = ca.chunk_attn_mixed_fwd(to_dev(Q), mode, k=to_dev(K), v=to_dev(V),
                                   kv_indptr=i32(indptr), kv_indices=i32(indices), kv_block=blk,
                                   kv_seg=seg, q_block=blk, q_seg=seg, k_flat=to_dev(Kf),
                                   v_flat=to_dev(Vf), cu_seqlens=i32(cu), cu_seqlens_host=cu,
                                   workspace=ws)
    torch.cuda.synchronize()
    assert _touched(ws), "balanced schedule not taken"
    sc = 1 / math.sqrt(d)
    for m in range(3):
        hs = [h for h in range(H) if mode[h] == m]
        if m == 0:
            Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc, heads=hs)
        elif m == 1:
            Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, indptr, indices, blk, seg, blk,
                                           seg, sc, heads=hs)
        else:
            Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, sc, heads=hs)
        assert_o(o[:, :, hs], Or, True, f"balanced mixed mode {m}")
        assert_lse(l[:, hs], Lr, f"balanced mixed mode {m}")


@pytest.mark.parametrize("B,H,Nq,maxlen,seed", [
    (1, 300, 300, 2000, 13),    # 300 heads: two launches (at most 256 heads each)
    (2, 37, 513, 4000, 14),     # three query tiles, the last of one row
])
def test_balanced_many_short_heads(B, H, Nq, maxlen, seed):
    """Many short heads (0 to tens of key tiles, some empty) under the forced
    balanced schedule: runs cross many query tiles, so workgroup ranges start
    and end inside the per-tile cost charge, on tiny tiles and at key tails;
    the whole output is compared."""
    say(f"balanced many short heads B={B} H={H} Nq={Nq} maxlen={maxlen}")
    d = 64
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, maxlen + 1, size=B * H)
    lens[rng.integers(0, B * H, size=3)] = 0
    cu = np.zeros(B * H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    Q = _gen(seed + 1, (B, Nq, H, d), 1.2)
    Kf, Vf = _gen(seed + 2, (int(cu[-1]), d), 1.2), _gen(seed + 3, (int(cu[-1]), d))
    ws = _nan_ws(d)
    o, l = ca.chunk_attn_varlen_fwd(to_dev(Q), to_dev(Kf), to_dev(Vf), i32(cu),
                                    cu_seqlens_host=cu, balanced="always", workspace=ws,
                                    out=nan_out(B, Nq, H, d), lse=nan_lse(B, H, Nq))
    torch.cuda.synchronize()
    assert _touched(ws), "balanced schedule not taken"
    assert_written("balanced many short heads", o, l)
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, 1 / math.sqrt(d))
    assert_o(o, Or, True, "balanced many short heads")
    assert_lse(l, Lr, "balanced many short heads")


def test_workspace_too_small_is_rejected():
    say("workspace too small")
    B, H, Nq, Nkv, d = 1, 2, 256, 8192, 128
    q = torch.zeros((B, Nq, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Nkv, H, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        ca.chunk_attn_fwd(q, k, k, workspace=ws)


def test_balanced_forced_on_the_wan_layer():
    say("balanced schedule forced on the Wan dense layer")
    w = wl.wan_dense(seed=0)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    ws = _nan_ws(w.d)
    o, l = nan_out(1, w.Nq, w.H, w.d), nan_lse(1, w.H, w.Nq)
    ca.chunk_attn_fwd(q, k, v, scale=w.scale, balanced="always", workspace=ws, out=o, lse=l)
    torch.cuda.synchronize()
    assert _touched(ws), "balanced schedule not taken"
    assert_written("wan balanced", o, l)
    rows = wave_rows(w.Nq, seed=7)
    Or, Lr = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale, rows=rows)
    assert_o(o[:, rows], Or, True, "wan balanced")
    assert_lse(l[:, :, rows], Lr, "wan balanced")

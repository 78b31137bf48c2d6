"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the calls launch kernels only (no allocation, memset, copy or
synchronisation inside the library), so a serving loop can capture a whole
layer once and replay it.  One graph holds the dense call under the balanced
schedule (attention + split merge on a workspace), the ragged call, the
local/history branches with their LSE merge, the whole block-sparse path
(block means, selections and block lists, one-pass PBSA) and the mixed call.
Each of three replays, with eager launches and synchronisations between
them, must reproduce the eager outputs bit for bit; the eager outputs are
themselves checked against the CPU oracle on sampled rows."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
import oracle as orc
from kv_cache_attention_chunk_amd import workloads as wl
from helpers import assert_lse, assert_o, i32, to_dev

pytestmark = pytest.mark.gpu

B, H, NQ, D = 1, 4, 600, 128
SEG = 1560                      # frame-aligned 64-token blocks, 25 per frame
NKV = 3 * SEG


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _gen(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * scale)


def test_graph_capture_and_replay():
    say(f"graph capture and replay: B={B} H={H} Nq={NQ} Nkv={NKV} d={D}")
    sc = 1 / math.sqrt(D)
    Q, K, V = _gen(1, (B, NQ, H, D), 1.2), _gen(2, (B, NKV, H, D), 1.2), _gen(3, (B, NKV, H, D))
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    # ragged heads: per-head frame counts, flat K/V
    lens = np.array([SEG, 3 * SEG, 2 * SEG - 100, 500])
    cu = np.zeros(B * H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    Kf, Vf = _gen(4, (int(cu[-1]), D)), _gen(5, (int(cu[-1]), D))
    kf, vf, cu_d = to_dev(Kf), to_dev(Vf), i32(cu)
    # local / history branches: per-head block lists (one query block = the chunk)
    nkb = orc.block_spans(NKV, 64, SEG).shape[0]
    local = np.concatenate([np.arange(25), np.arange(50, nkb)]).astype(np.int32)
    hist = np.arange(25, 50, dtype=np.int32)
    br = [(i32(np.arange(B * H + 1) * len(x)), i32(np.tile(x, B * H))) for x in (local, hist)]
    # block-sparse path: sink frame 0, history frame 1 (C = 8), local frame 2 (K = 5)
    sp = dict(sink_begin=0, sink_count=25, hist_begin=25, hist_count=25, C=8, local_begin=50,
              local_count=25, K=5)
    sp_ws = torch.empty(ca.block_sparse_workspace(B, H, NQ, NKV, D, block=64, seg=SEG,
                                                  have_k_mean=False, **sp).bytes,
                        dtype=torch.uint8, device="cuda")
    # mixed: dense / ragged / block-list heads
    mode = np.array([0, 2, 1, 2], np.int32)
    nqb = ca.num_blocks(NQ, 64, SEG)
    mip, mix = wl.random_csr(np.random.default_rng(6), B * H * nqb, nkb, 12)
    mip_d, mix_d = i32(mip), i32(mix)        # device copies made before any capture
    ws_d, ws_r, ws_m = (torch.empty(ca.workspace_bytes(D), dtype=torch.uint8, device="cuda")
                        for _ in range(3))

    outs = {}

    def buf(name, *shape, dtype=torch.float32):
        outs[name] = torch.empty(shape, dtype=dtype, device="cuda")
        return outs[name]

    o_d, l_d = buf("o_dense", B, NQ, H, D, dtype=torch.bfloat16), buf("l_dense", B, H, NQ)
    o_r, l_r = buf("o_ragged", B, NQ, H, D, dtype=torch.bfloat16), buf("l_ragged", B, H, NQ)
    o_b = [buf(f"o_br{i}", B, NQ, H, D) for i in range(2)]
    l_b = [buf(f"l_br{i}", B, H, NQ) for i in range(2)]
    o_mg, l_mg = buf("o_merge", B, NQ, H, D, dtype=torch.bfloat16), buf("l_merge", B, H, NQ)
    o_s, l_s = buf("o_sparse", B, NQ, H, D, dtype=torch.bfloat16), buf("l_sparse", B, H, NQ)
    o_x, l_x = buf("o_mixed", B, NQ, H, D, dtype=torch.bfloat16), buf("l_mixed", B, H, NQ)

    def layer():
        ca.chunk_attn_fwd(q, k, v, scale=sc, out=o_d, lse=l_d, balanced="always", workspace=ws_d)
        ca.chunk_attn_varlen_fwd(q, kf, vf, cu_d, cu_seqlens_host=cu, scale=sc, out=o_r, lse=l_r,
                                 balanced="always", workspace=ws_r)
        for (ip, ix), ob, lb in zip(br, o_b, l_b):
            ca.chunk_attn_fwd(q, k, v, kv_indptr=ip, kv_indices=ix, kv_block=64, kv_seg=SEG,
                              q_block=NQ, q_seg=NQ, scale=sc, out_dtype=torch.float32, out=ob,
                              lse=lb)
        ca.lse_merge(o_b[0], l_b[0], o_b[1], l_b[1], out=o_mg, out_lse=l_mg)
        ca.block_sparse_fwd(q, k, v, block=64, seg=SEG, scale=sc, out=o_s, lse=l_s,
                            workspace=sp_ws, **sp)
        ca.chunk_attn_mixed_fwd(q, mode, k=k, v=v, kv_indptr=mip_d, kv_indices=mix_d,
                                kv_block=64, kv_seg=SEG, q_block=64, q_seg=SEG, k_flat=kf,
                                v_flat=vf, cu_seqlens=cu_d, cu_seqlens_host=cu, scale=sc, out=o_x,
                                lse=l_x, workspace=ws_m)

    # eager reference (also warms up every code path before the capture)
    layer()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}

    # the eager results are the attention the oracle defines (sampled rows)
    rows = np.unique(np.r_[0, 255, 256, 311, NQ - 1])
    Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc, rows=rows)
    assert_o(ref["o_dense"][:, rows], Or, True, "graph eager dense")
    assert_lse(ref["l_dense"][:, :, rows], Lr, "graph eager dense")
    assert_o(ref["o_merge"][:, rows], Or, True, "graph eager merge")
    assert_lse(ref["l_merge"][:, :, rows], Lr, "graph eager merge")
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, sc, rows=rows)
    assert_o(ref["o_ragged"][:, rows], Or, True, "graph eager ragged")
    assert_lse(ref["l_ragged"][:, :, rows], Lr, "graph eager ragged")

    # capture on a side stream, as torch requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()

    other = torch.empty_like(o_d)
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            same = torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                               ref[n].view(torch.int16) if t.dtype == torch.bfloat16
                               else ref[n].view(torch.int32))
            assert same, f"replay {rep}: {n} differs from the eager result"
        # eager work between replays, on other buffers
        ca.chunk_attn_fwd(k[:, :NQ], q, q, scale=sc, out=other)
        torch.cuda.synchronize()
    say("graph replays match the eager outputs bit for bit")

"""Run-to-run determinism and output guard bands on the GPU.

Every path is a fixed sequence of float32 operations per output element (no
atomics in the arithmetic, fixed reduction orders, a static work split), so
two calls on the same inputs must agree bit for bit: the balanced schedule
(split key ranges merged through the LSE), ragged heads, the block-sparse
pipeline, the dual-output pass, the latent-KV path and ragged packing.  The
guard-band tests write into views of larger buffers filled with a canary and
check that nothing outside the view changed."""
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


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _same(a, b, what):
    if a.dtype in (torch.bfloat16, torch.float16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b), f"{what}: two calls differ"


def _gen(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * scale)


def test_balanced_dense_is_deterministic():
    say("determinism: balanced dense")
    q = to_dev(_gen(1, (1, 700, 3, 128), 1.2))
    k = to_dev(_gen(2, (1, 9000, 3, 128), 1.2))
    v = to_dev(_gen(3, (1, 9000, 3, 128)))
    runs = [ca.chunk_attn_fwd(q, k, v, balanced="always") for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(2):
        _same(runs[0][i], runs[1][i], "balanced dense")


def test_ragged_wan_is_deterministic():
    say("determinism: ragged 12-head layer (balanced schedule)")
    w = wl.ragged(seed=0)
    q, kf, vf, cu = to_dev(w.q), to_dev(w.k_flat), to_dev(w.v_flat), i32(w.cu_seqlens)
    runs = [ca.chunk_attn_varlen_fwd(q, kf, vf, cu, cu_seqlens_host=w.cu_seqlens, scale=w.scale)
            for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(2):
        _same(runs[0][i], runs[1][i], "ragged")


def test_block_sparse_wan_is_deterministic():
    say("determinism: block-sparse pipeline at the Wan shape, K = 10")
    w = wl.wan_dense(seed=0)
    lay = wl.sparse_layout(w, 0.125)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    args = dict(sink_begin=0, sink_count=lay["sink_count"], hist_begin=lay["hist_begin"],
                hist_count=lay["hist_count"], C=lay["C"], local_begin=lay["local_begin"],
                local_count=lay["local_count"], K=lay["K"], block=64, seg=1560, scale=w.scale)
    r0 = ca.block_sparse_fwd(q, k, v, **args)
    r1 = ca.block_sparse_fwd(q, k, v, **args)
    torch.cuda.synchronize()
    _same(r0[0], r1[0], "sparse O")
    _same(r0[1], r1[1], "sparse LSE")
    for key in ("persistent", "local", "local_indices", "shared_indices"):
        assert torch.equal(r0[2][key], r1[2][key]), key


def test_dual_is_deterministic():
    say("determinism: dual-output pass")
    B, H, Nq, Nkv, d, seg = 1, 3, 500, 3000, 128, 1000
    q, k, v = (to_dev(_gen(s, (B, n, H, d), 1.3)) for s, n in ((4, Nq), (5, Nkv), (6, Nkv)))
    nkb = orc.block_spans(Nkv, 64, seg).shape[0]
    rng = np.random.default_rng(2)
    lists = [rng.permutation(nkb)[:30] for _ in range(B * H)]
    ip = i32(np.arange(B * H + 1) * 30)
    ix = i32(np.concatenate(lists))
    runs = [ca.chunk_attn_dual_fwd(q, k, v, ip, ix, 12, kv_block=64, kv_seg=seg, q_block=Nq,
                                   q_seg=Nq) for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(4):
        _same(runs[0][i], runs[1][i], f"dual output {i}")


def test_mla_is_deterministic():
    say("determinism: latent-KV path")
    rng = np.random.default_rng(9)
    B, Nq, H, N = 1, 300, 12, 2000
    q = to_dev(wl.Bf16Tensor.from_f32(rng.standard_normal((B, Nq, H, 128), dtype=np.float32)))
    kv = ca.cast_bf16_to_f16(to_dev(wl.Bf16Tensor.from_f32(
        rng.standard_normal((B, N, 224), dtype=np.float32))))
    wk = to_dev(wl.Bf16Tensor.from_f32(rng.standard_normal((H, 96, 192), dtype=np.float32) / 14))
    wv = to_dev(wl.Bf16Tensor.from_f32(rng.standard_normal((H, 128, 192), dtype=np.float32) / 14))
    runs = [ca.mla_chunk_attn(q, kv, wk, wv) for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(3):
        _same(runs[0][i], runs[1][i], f"mla output {i}")


def test_pack_guard_bands_and_determinism():
    say("pack: guard bands around the flat outputs, two calls bit-equal")
    rng = np.random.default_rng(11)
    B, H, T, nf, d = 1, 4, 50, 6, 128
    K = wl.Bf16Tensor.from_f32(rng.standard_normal((B, nf * T, H, d), dtype=np.float32))
    V = wl.Bf16Tensor.from_f32(rng.standard_normal((B, nf * T, H, d), dtype=np.float32))
    frames = [[0, (1, 2), 5], [3], [(4, 5), 0], [1, 2, 3, 4]]
    k, v = to_dev(K), to_dev(V)
    rows = sum(len(f) for f in frames) * T
    outs = []
    for _ in range(2):
        kb = torch.full((rows * d + 2048,), -7.0, dtype=torch.bfloat16, device="cuda")
        vb = torch.full((rows * d + 2048,), 9.0, dtype=torch.bfloat16, device="cuda")
        cb = torch.full((B * H + 1 + 64,), -5, dtype=torch.int32, device="cuda")
        kf, vf = kb[1024:1024 + rows * d].view(rows, d), vb[1024:1024 + rows * d].view(rows, d)
        cu = cb[32:32 + B * H + 1]
        ca.pack_ragged(k, v, frames, T, out_k=kf, out_v=vf, out_cu=cu)
        torch.cuda.synchronize()
        for buf, val, n in ((kb, -7.0, 1024), (vb, 9.0, 1024), (cb, -5, 32)):
            assert torch.all(buf[:n] == val) and torch.all(buf[-n:] == val), "guard band written"
        outs.append((kf.clone(), vf.clone(), cu.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    ptr = np.zeros(B * H + 1, np.int64)
    src = []
    for bh, fl in enumerate(frames):
        for f in fl:
            src.append(tuple(f) if isinstance(f, tuple) else (f, -1))
        ptr[bh + 1] = len(src)
    rk, rv, rcu = orc.pack_ragged(K.bits, V.bits, ptr, np.array(src), T)
    assert np.array_equal(outs[0][0].view(torch.int16).cpu().numpy().view(np.uint16), rk)
    assert np.array_equal(outs[0][1].view(torch.int16).cpu().numpy().view(np.uint16), rv)
    assert np.array_equal(outs[0][2].cpu().numpy(), rcu)


@pytest.mark.parametrize("balanced", ["never", "always"])
def test_varlen_guard_bands(balanced):
    say(f"varlen: guard bands around O and LSE, split policy {balanced}")
    rng = np.random.default_rng(12)
    B, H, Nq, d = 1, 3, 300, 128
    lens = [0, 5000, 777]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Q = wl.Bf16Tensor.from_f32(rng.standard_normal((B, Nq, H, d), dtype=np.float32))
    Kf = wl.Bf16Tensor.from_f32(rng.standard_normal((int(cu[-1]), d), dtype=np.float32))
    Vf = wl.Bf16Tensor.from_f32(rng.standard_normal((int(cu[-1]), d), dtype=np.float32))
    n = B * Nq * H * d
    ob = torch.full((n + 4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((B * H * Nq + 256,), -2.0, dtype=torch.float32, device="cuda")
    o = ob[2048:2048 + n].view(B, Nq, H, d)
    l = lb[128:128 + B * H * Nq].view(B, H, Nq)
    ca.chunk_attn_varlen_fwd(to_dev(Q), to_dev(Kf), to_dev(Vf), i32(cu), cu_seqlens_host=cu,
                             out=o, lse=l, balanced=balanced)
    torch.cuda.synchronize()
    assert torch.all(ob[:2048] == 3.0) and torch.all(ob[-2048:] == 3.0), "O guard band written"
    assert torch.all(lb[:128] == -2.0) and torch.all(lb[-128:] == -2.0), "LSE guard band written"
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, 1 / math.sqrt(d))
    assert_o(o, Or, True, "varlen guard")
    assert_lse(l, Lr, "varlen guard")

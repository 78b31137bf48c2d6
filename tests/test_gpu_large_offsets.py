"""GPU parity at the largest strides the library accepts: caches, queries and
outputs whose element offsets pass 2^31 (about 4 GiB of bf16), so that every
address product in the kernels must be formed in 64 bits.

Two layouts, each checked against the CPU oracle on the whole output (O
max-abs 1e-2, LSE max-abs 1e-3):
  * a key/value cache with the maximal row stride, 2^23 elements: 300 keys
    (four 64-key tiles and a 44-key tail) reach element 299 * 2^23, about
    2.5e9; dense, balanced split, block lists, one-pass PBSA, ragged and block
    means read it;
  * a batch stride of 2^31 + 64 elements on K, V, Q and O alike: batch 1
    lives past element 2^31 in every tensor; dense, block lists, PBSA, the
    LSE merge (with its inputs and output there too) and block means.
Each layout is one allocation of 4.3-5 GB; only the rows the views cover
are written.
"""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
import oracle as orc
from kv_cache_attention_chunk_amd import workloads as wl
from helpers import assert_lse, assert_o, assert_written, i32, nan_lse, nan_out, to_dev

pytestmark = pytest.mark.gpu

ROW_STRIDE_MAX = 1 << 23          # the largest K/V row stride the entry points accept
BIG_BATCH_STRIDE = (1 << 31) + 64


@pytest.fixture(autouse=True)
def _release():
    """Hand each test's multi-GB buffer back to the device once it is done."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _gen(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * scale)


def _csr(rows):
    ip = np.zeros(len(rows) + 1, np.int32)
    ip[1:] = np.cumsum([len(r) for r in rows])
    ix = np.concatenate(rows).astype(np.int32) if ip[-1] else np.zeros(1, np.int32)
    return ip, ix


def _pbsa_lists(rng, BH, nqb, nkb, n_shared, n_local):
    """Per head a shared list holding the last block (the farthest keys), per
    (head, query block) a disjoint local list; returns both CSRs and the
    union CSR the oracle attends over."""
    shared, local = [], []
    for _ in range(BH):
        rest = rng.permutation(nkb - 1)
        sh = np.concatenate([[nkb - 1], rest[:n_shared - 1]])
        shared.append(sh)
        for _ in range(nqb):
            local.append(rng.permutation(rest[n_shared - 1:])[:n_local])
    union = [np.concatenate([shared[r // nqb], local[r]]) for r in range(len(local))]
    return _csr(shared), _csr(local), _csr(union)


def _view(buf, shape, strides, offset):
    """A strided view into `buf`; torch rejects one that leaves the storage."""
    v = buf.as_strided(shape, strides, offset)
    last = offset + sum((n - 1) * s for n, s in zip(shape, strides))
    assert last < buf.numel()
    return v


def test_max_row_stride_cache_past_2g_elements():
    B, H, Nq, Nkv, d, RS = 1, 2, 130, 300, 128, ROW_STRIDE_MAX
    say(f"row stride 2^23: B={B} H={H} Nq={Nq} Nkv={Nkv} d={d}")
    Q, K, V = _gen(1, (B, Nq, H, d), 1.3), _gen(2, (B, Nkv, H, d), 1.3), _gen(3, (B, Nkv, H, d))
    buf = torch.empty(Nkv * RS, dtype=torch.bfloat16, device="cuda")
    # row n of the cache: K heads at [n RS, n RS + H d), V heads right after
    k = _view(buf, (B, Nkv, H, d), (Nkv * RS, RS, d, 1), 0)
    v = _view(buf, (B, Nkv, H, d), (Nkv * RS, RS, d, 1), H * d)
    assert (Nkv - 1) * RS > 2 ** 31
    k.copy_(to_dev(K))
    v.copy_(to_dev(V))
    q = to_dev(Q)
    sc = 1 / math.sqrt(d)
    Od, Ld = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc)
    for policy in ("never", "always"):
        say(f"row stride 2^23: dense, split {policy}")
        o, l = ca.chunk_attn_fwd(q, k, v, balanced=policy, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_o(o, Od, False, f"row stride dense {policy}")
        assert_lse(l, Ld, f"row stride dense {policy}")

    # block lists: 5 key blocks over one 300-token segment (64 x 4 + 44),
    # 3 query blocks (64, 64, 2); every list holds the 44-key tail block
    say("row stride 2^23: block lists")
    rng = np.random.default_rng(7)
    nkb, nqb = 5, 3
    rows = [np.concatenate([[4], rng.permutation(4)[:rng.integers(0, 5)]]) for _ in range(B * H * nqb)]
    ip, ix = _csr(rows)
    o, l = ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip), kv_indices=i32(ix), kv_block=64,
                             kv_seg=Nkv, q_block=64, q_seg=Nq)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, ip, ix, 64, Nkv, 64, Nq, sc)
    assert_o(o, Or, True, "row stride blocks")
    assert_lse(l, Lr, "row stride blocks")

    say("row stride 2^23: one-pass PBSA")
    (sp, sx), (lp, lx), (up, ux) = _pbsa_lists(rng, B * H, nqb, nkb, 2, 2)
    o, l = nan_out(B, Nq, H, d, torch.float32), nan_lse(B, H, Nq)
    ca.chunk_attn_pbsa_fwd(q, k, v, i32(sp), i32(sx), i32(lp), i32(lx), kv_block=64,
                           kv_seg=Nkv, q_block=64, q_seg=Nq, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("row stride pbsa", o, l)
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, up, ux, 64, Nkv, 64, Nq, sc)
    assert_o(o, Or, False, "row stride pbsa")
    assert_lse(l, Lr, "row stride pbsa")

    # ragged: the 300 rows of head 0 as a flat cache, split 170 / 130
    # between the two heads
    kf = _view(buf, (Nkv, d), (RS, 1), 0)
    vf = _view(buf, (Nkv, d), (RS, 1), H * d)
    cu = np.array([0, 170, Nkv], np.int32)
    Kf, Vf = K.f32[0, :, 0], V.f32[0, :, 0]
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf, Vf, cu, sc)
    for host in (False, True):
        say(f"row stride 2^23: ragged, host boundaries {host}")
        o, l = ca.chunk_attn_varlen_fwd(q, kf, vf, i32(cu), cu_seqlens_host=cu if host else None,
                                        out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_o(o, Or, False, f"row stride ragged host={host}")
        assert_lse(l, Lr, f"row stride ragged host={host}")

    say("row stride 2^23: block means")
    m = ca.block_mean(k, 64, Nkv)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().numpy(), orc.block_mean(K.f32, 64, Nkv), rtol=0, atol=2e-6)


def test_batch_stride_past_2g_elements():
    B, H, Nq, Nkv, d, SB = 2, 2, 100, 200, 64, BIG_BATCH_STRIDE
    say(f"batch stride 2^31+64: B={B} H={H} Nq={Nq} Nkv={Nkv} d={d}")
    Q, K, V = _gen(11, (B, Nq, H, d), 1.3), _gen(12, (B, Nkv, H, d), 1.3), _gen(13, (B, Nkv, H, d))
    S, Sq = Nkv * H * d, Nq * H * d
    # batch b's tensors sit at b SB + (K 0, V S, Q 2S, then five Q-sized outputs)
    buf = torch.empty(SB + 2 * S + 6 * Sq, dtype=torch.bfloat16, device="cuda")
    kst, qst = (SB, H * d, d, 1), (SB, H * d, d, 1)
    k = _view(buf, (B, Nkv, H, d), kst, 0)
    v = _view(buf, (B, Nkv, H, d), kst, S)
    q = _view(buf, (B, Nq, H, d), qst, 2 * S)
    outs = [_view(buf, (B, Nq, H, d), qst, 2 * S + (1 + i) * Sq) for i in range(5)]
    k.copy_(to_dev(K))
    v.copy_(to_dev(V))
    q.copy_(to_dev(Q))
    for t in outs:
        t.fill_(float("nan"))
    sc = 1 / math.sqrt(d)
    say("batch stride: dense")
    Od, Ld = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc)
    o, l = ca.chunk_attn_fwd(q, k, v, out=outs[0])
    torch.cuda.synchronize()
    assert_o(o, Od, True, "batch stride dense")
    assert_lse(l, Ld, "batch stride dense")

    # two branches over the keys [0, 120) and [120, 200), then their merge
    say("batch stride: branches and LSE merge")
    o1, l1 = ca.chunk_attn_fwd(q, k[:, :120], v[:, :120], out=outs[1])
    o2, l2 = ca.chunk_attn_fwd(q, k[:, 120:], v[:, 120:], out=outs[2])
    om, lm = ca.lse_merge(o1, l1, o2, l2, out=outs[3])
    torch.cuda.synchronize()
    O1, L1 = orc.chunk_attn_dense(Q.f32, K.f32[:, :120], V.f32[:, :120], sc)
    assert_o(o1, O1, True, "batch stride branch 1")
    assert_lse(l1, L1, "batch stride branch 1")
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    Om, Lm = orc.lse_merge_bshd(f64(o1), f64(l1), f64(o2), f64(l2))
    assert_o(om, Om, True, "batch stride merge")
    assert_lse(lm, Lm, "batch stride merge")

    say("batch stride: block lists")
    nkb, nqb = orc.block_spans(Nkv, 64, Nkv).shape[0], orc.block_spans(Nq, 64, Nq).shape[0]
    rng = np.random.default_rng(17)
    ip, ix = wl.random_csr(rng, B * H * nqb, nkb, nkb)
    o, l = ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip),
                             kv_indices=i32(ix if len(ix) else np.zeros(1)), kv_block=64,
                             kv_seg=Nkv, q_block=64, q_seg=Nq, out=outs[4])
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, ip, ix, 64, Nkv, 64, Nq, sc)
    assert_o(o, Or, True, "batch stride blocks")
    assert_lse(l, Lr, "batch stride blocks")

    say("batch stride: one-pass PBSA")
    (sp, sx), (lp, lx), (up, ux) = _pbsa_lists(rng, B * H, nqb, nkb, 2, 1)
    outs[0].fill_(float("nan"))
    l = nan_lse(B, H, Nq)
    o, _ = ca.chunk_attn_pbsa_fwd(q, k, v, i32(sp), i32(sx), i32(lp), i32(lx), kv_block=64,
                                  kv_seg=Nkv, q_block=64, q_seg=Nq, out=outs[0], lse=l)
    torch.cuda.synchronize()
    assert_written("batch stride pbsa", o, l)
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, up, ux, 64, Nkv, 64, Nq, sc)
    assert_o(o, Or, True, "batch stride pbsa")
    assert_lse(l, Lr, "batch stride pbsa")

    say("batch stride: block means")
    m = ca.block_mean(v, 64, Nkv)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().numpy(), orc.block_mean(V.f32, 64, Nkv), rtol=0, atol=2e-6)

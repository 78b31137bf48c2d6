"""GPU parity: every HIP kernel against the CPU oracle on the same seeded
inputs (O max-abs 1e-2, LSE max-abs 1e-3, block ids exact except near-ties).

Small cases span several 64-key tiles, ragged query/key tails, 24-token tail
blocks, empty key sets, d = 64 and 128 and strided head-subset views; the
workload-sized cases run the library exactly as the benchmark does, start
from NaN-filled outputs that every element must overwrite, and are checked on
the whole layer (dense) or on a row of every 32-row wave slice of every
workgroup, for every head.
"""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
from kv_cache_attention_chunk_amd import workloads as wl
import oracle as orc
from helpers import (assert_lse, assert_o, assert_written, compare_topk, i32, nan_lse,
                     nan_out, to_dev, wave_rows)

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _loaded():
    from kv_cache_attention_chunk_amd import _lib
    _lib.lib()          # raises if the HIP library is missing


def _gen(seed, B, N, H, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.Bf16Tensor.from_f32(rng.standard_normal((B, N, H, d), dtype=np.float32) * scale)


# ---------------------------------------------------------------------------
# workload of the tiny dense chunk (256 q vs 1024 kv, 2 heads, d 64)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tiny_dense(out_dtype):
    say(f"tiny dense {out_dtype}")
    w = wl.tiny_dense(seed=0)
    o, l = ca.chunk_attn_fwd(to_dev(w.q), to_dev(w.k), to_dev(w.v), scale=w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale)
    assert_o(o, Or, out_dtype == torch.bfloat16, "tiny dense")
    assert_lse(l, Lr, "tiny dense")


@pytest.mark.parametrize("q_block", [64, 256])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_local_history_merge(q_block, seed):
    say(f"tiny local/history merge q_block={q_block} seed={seed}")
    w = wl.tiny_dense(seed=seed)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    nqb = w.Nq // q_block
    rows = w.B * w.H * nqb
    branches = []
    for blocks in (w.meta["local_blocks"], w.meta["history_blocks"]):
        indptr = np.arange(rows + 1, dtype=np.int32) * len(blocks)
        indices = np.tile(np.array(blocks, np.int32), rows)
        o, l = ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(indptr), kv_indices=i32(indices),
                                 kv_block=64, kv_seg=w.Nkv, q_block=q_block, q_seg=w.Nq,
                                 scale=w.scale, out_dtype=torch.float32)
        Or, Lr = orc.chunk_attn_blocks(w.q.f32, w.k.f32, w.v.f32, indptr, indices, 64, w.Nkv,
                                       q_block, w.Nq, w.scale)
        torch.cuda.synchronize()
        assert_o(o, Or, False, "branch")
        assert_lse(l, Lr, "branch")
        branches.append((o, l))
    om, lm = ca.lse_merge(branches[0][0], branches[0][1], branches[1][0], branches[1][1],
                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Od, Ld = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale)
    assert_o(om, Od, True, "merged vs dense")
    assert_lse(lm, Ld, "merged vs dense")


# ---------------------------------------------------------------------------
# dense mode: ragged sizes, d 64 / 128, batch > 1, strided views, empty caches
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,Nq,Nkv,d,sc", [
    (2, 3, 200, 1000, 128, 1.0), (1, 2, 129, 63, 64, 1.5), (1, 1, 33, 1, 128, 2.0),
    (1, 2, 64, 0, 64, 1.0), (2, 2, 300, 777, 64, 0.7), (1, 3, 1, 130, 128, 1.0),
])
def test_dense_shapes(B, H, Nq, Nkv, d, sc):
    say(f"dense B={B} H={H} Nq={Nq} Nkv={Nkv} d={d}")
    Q, K, V = _gen(1, B, Nq, H, d, sc), _gen(2, B, Nkv, H, d, sc), _gen(3, B, Nkv, H, d)
    o, l = ca.chunk_attn_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, 1 / math.sqrt(d))
    assert_o(o, Or, True, "dense")
    assert_lse(l, Lr, "dense")


def test_dense_strided_head_subset_views():
    say("dense strided views")
    B, Nq, Nkv, H, d = 1, 150, 300, 6, 128
    Q, K, V = _gen(4, B, Nq, H, d), _gen(5, B, Nkv, H, d), _gen(6, B, Nkv, H, d)
    q, k, v = to_dev(Q)[:, :, 1::2], to_dev(K)[:, :, 1::2], to_dev(V)[:, :, 1::2]
    out = torch.full((B, Nq, 5, d), 7.0, dtype=torch.float32, device="cuda")
    o, l = ca.chunk_attn_fwd(q, k, v, out=out[:, :, 1:4], out_dtype=torch.float32)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_dense(Q.f32[:, :, 1::2], K.f32[:, :, 1::2], V.f32[:, :, 1::2], 1 / math.sqrt(d))
    assert_o(o, Or, False, "strided")
    assert_lse(l, Lr, "strided")
    assert torch.all(out[:, :, 0] == 7.0) and torch.all(out[:, :, 4] == 7.0)


def test_dense_output_guard_bands_and_determinism():
    say("dense guard bands + determinism")
    B, Nq, Nkv, H, d = 1, 130, 200, 2, 64
    Q, K, V = _gen(7, B, Nq, H, d), _gen(8, B, Nkv, H, d), _gen(9, B, Nkv, H, d)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    buf = torch.full((B * Nq * H * d + 2048,), -3.0, dtype=torch.bfloat16, device="cuda")
    o = buf[1024:1024 + B * Nq * H * d].view(B, Nq, H, d)
    lbuf = torch.full((B * H * Nq + 128,), 5.0, dtype=torch.float32, device="cuda")
    lse = lbuf[64:64 + B * H * Nq].view(B, H, Nq)
    ca.chunk_attn_fwd(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == -3.0) and torch.all(buf[-1024:] == -3.0)
    assert torch.all(lbuf[:64] == 5.0) and torch.all(lbuf[-64:] == 5.0)
    o2, l2 = ca.chunk_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


# ---------------------------------------------------------------------------
# block-list mode (PBSA): frame-aligned tiling with tail blocks, empty rows
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,seed", [(128, 0), (64, 1), (128, 2)])
def test_blocks_random_lists(d, seed):
    say(f"blocks random lists d={d} seed={seed}")
    B, H, Nq, Nkv, seg, blk = 2, 2, 200, 500, 100, 64      # tiles of 64 + 36 per segment
    Q, K, V = _gen(10 + seed, B, Nq, H, d), _gen(20 + seed, B, Nkv, H, d), _gen(30 + seed, B, Nkv, H, d)
    nkb = orc.block_spans(Nkv, blk, seg).shape[0]
    nqb = orc.block_spans(Nq, blk, seg).shape[0]
    rng = np.random.default_rng(seed)
    indptr, indices = wl.random_csr(rng, B * H * nqb, nkb, nkb)
    o, l = ca.chunk_attn_fwd(to_dev(Q), to_dev(K), to_dev(V), kv_indptr=i32(indptr),
                             kv_indices=i32(indices if len(indices) else np.zeros(1)),
                             kv_block=blk, kv_seg=seg, q_block=blk, q_seg=seg)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, indptr, indices, blk, seg, blk, seg,
                                   1 / math.sqrt(d))
    assert_o(o, Or, True, "blocks")
    assert_lse(l, Lr, "blocks")


def test_blocks_unsorted_lists_and_small_blocks():
    say("blocks unsorted lists, 24-token blocks")
    B, H, Nq, Nkv, d = 1, 3, 96, 480, 128
    Q, K, V = _gen(41, B, Nq, H, d), _gen(42, B, Nkv, H, d), _gen(43, B, Nkv, H, d)
    blk, seg = 24, 480
    nkb = Nkv // blk
    rng = np.random.default_rng(3)
    lists = [rng.permutation(nkb)[:rng.integers(0, nkb)] for _ in range(B * H * 4)]
    indptr = np.zeros(len(lists) + 1, np.int32)
    indptr[1:] = np.cumsum([len(x) for x in lists])
    indices = np.concatenate(lists).astype(np.int32)
    o, l = ca.chunk_attn_fwd(to_dev(Q), to_dev(K), to_dev(V), kv_indptr=i32(indptr),
                             kv_indices=i32(indices), kv_block=blk, kv_seg=seg, q_block=24, q_seg=Nq)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, indptr, indices, blk, seg, 24, Nq, 1 / math.sqrt(d))
    assert_o(o, Or, True, "blocks unsorted")
    assert_lse(l, Lr, "blocks unsorted")


# ---------------------------------------------------------------------------
# ragged mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("host_cu", [False, True])
def test_varlen_small(host_cu):
    say(f"varlen small host_cu={host_cu}")
    w = wl.ragged(seed=5, H=5, d=128, frames_q=2, frames_kv=21, frame_tokens=40)
    cu = w.cu_seqlens.copy()
    # make head 1 empty and head 3 end on a ragged length
    lens = np.diff(cu)
    lens[1] = 0
    lens[3] = 77
    cu2 = np.zeros_like(cu)
    cu2[1:] = np.cumsum(lens)
    Kf = wl.Bf16Tensor(w.k_flat.bits[:cu2[-1]].copy())
    Vf = wl.Bf16Tensor(w.v_flat.bits[:cu2[-1]].copy())
    o, l = ca.chunk_attn_varlen_fwd(to_dev(w.q), to_dev(Kf), to_dev(Vf), i32(cu2),
                                    cu_seqlens_host=cu2 if host_cu else None)
    torch.cuda.synchronize()
    Or, Lr = orc.chunk_attn_varlen(w.q.f32, Kf.f32, Vf.f32, cu2, w.scale)
    assert_o(o, Or, True, "varlen")
    assert_lse(l, Lr, "varlen")


def test_mixed_small():
    say("mixed small")
    w = wl.mixed(seed=3, H=6, d=64, frames_q=2, frames_kv=8, frame_tokens=100, topk_ratio=0.5)
    lay = dict(w.meta["sparse"])
    lay["C"] = 3
    sel = orc.sparse_selection(w.q.f32, w.k.f32, w.q_block, w.q_seg, w.kv_block, w.kv_seg, lay)
    o, l = ca.chunk_attn_mixed_fwd(
        to_dev(w.q), w.head_mode, k=to_dev(w.k), v=to_dev(w.v), kv_indptr=i32(sel["indptr"]),
        kv_indices=i32(sel["indices"]), kv_block=64, kv_seg=100, q_block=64, q_seg=100,
        k_flat=to_dev(w.k_flat), v_flat=to_dev(w.v_flat), cu_seqlens=i32(w.cu_seqlens),
        cu_seqlens_host=w.cu_seqlens)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    lg = l.cpu().numpy()
    for h in range(w.H):
        if w.head_mode[h] == 0:
            Or, Lr = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale, heads=[h])
        elif w.head_mode[h] == 1:
            Or, Lr = orc.chunk_attn_blocks(w.q.f32, w.k.f32, w.v.f32, sel["indptr"], sel["indices"],
                                           64, 100, 64, 100, w.scale, heads=[h])
        else:
            Or, Lr = orc.chunk_attn_varlen(w.q.f32, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens,
                                           w.scale, heads=[h])
        assert_o(torch.from_numpy(og[:, :, h:h + 1]), Or, True, f"mixed head {h}")
        assert_lse(torch.from_numpy(lg[:, h:h + 1]), Lr, f"mixed head {h}")


# ---------------------------------------------------------------------------
# LSE merge kernel
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("idt,odt", [(torch.float32, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                     (torch.float32, torch.float32), (torch.bfloat16, torch.float32)])
def test_lse_merge_kernel(idt, odt):
    say(f"lse_merge {idt}->{odt}")
    rng = np.random.default_rng(9)
    B, N, H, d = 2, 37, 3, 128
    o1 = torch.from_numpy(rng.standard_normal((B, N, H, d), dtype=np.float32)).to(idt).cuda()
    o2 = torch.from_numpy(rng.standard_normal((B, N, H, d), dtype=np.float32)).to(idt).cuda()
    l1 = rng.standard_normal((B, H, N)).astype(np.float32) * 5
    l2 = rng.standard_normal((B, H, N)).astype(np.float32) * 5
    l1[0, 0, :4] = -np.inf
    l2[0, 0, 2:6] = -np.inf
    l2[1, 2, 7] = l1[1, 2, 7]
    o, l = ca.lse_merge(o1, torch.from_numpy(l1).cuda(), o2, torch.from_numpy(l2).cuda(), out_dtype=odt)
    torch.cuda.synchronize()
    Or, Lr = orc.lse_merge_bshd(o1.float().cpu().numpy(), l1, o2.float().cpu().numpy(), l2)
    assert_o(o, Or, odt == torch.bfloat16, "merge")
    assert_lse(l, Lr, "merge")
    # in place into o1 / lse1
    if idt == odt:
        lt = torch.from_numpy(l1).cuda()
        ca.lse_merge(o1, lt, o2, torch.from_numpy(l2).cuda(), out=o1, out_lse=lt)
        torch.cuda.synchronize()
        assert torch.equal(o1.float(), o.float()) and torch.equal(lt, l)


# ---------------------------------------------------------------------------
# block means, scores + top-K, block lists
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,N,seg", [(128, 1560 * 2, 1560), (64, 300, 100), (128, 100, 100)])
def test_block_mean_kernel(d, N, seg):
    say(f"block_mean d={d} N={N} seg={seg}")
    X = _gen(50, 2, N, 3, d, 2.0)
    m = ca.block_mean(to_dev(X), 64, seg)
    torch.cuda.synchronize()
    ref = orc.block_mean(X.f32, 64, seg)
    np.testing.assert_allclose(m.cpu().numpy(), ref, rtol=0, atol=2e-6)


def test_topk_planted_ties_and_full():
    say("topk planted")
    d = 128
    q = np.zeros((1, 2, 3, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 2, 90, d), np.float32)
    rng = np.random.default_rng(0)
    k[..., 0] = rng.integers(0, 20, size=(1, 2, 90)).astype(np.float32)   # many exact ties
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda()
    for K, cb, cc in [(5, 10, 75), (1, 0, 90), (75, 15, 75), (32, 3, 80)]:
        idx, sc = ca.block_score_topk(qt, kt, K, cand_begin=cb, cand_count=cc, return_scores=True)
        torch.cuda.synchronize()
        ref = orc.block_score_topk(q, k, cb, cc, K)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])     # exact ties: lower id wins
        np.testing.assert_array_equal(sc.cpu().numpy(), ref["score"])


@pytest.mark.parametrize("n,K", [(129, 5), (200, 17), (425, 32), (2000, 100), (3000, 2999),
                                 (4096, 1), (4096, 4096)])
def test_topk_radix_select_planted_ties(n, K):
    """Candidate sets above 128 take the radix select (256- and 1024-thread
    workgroups): ids and scores exact against the oracle with many exact
    ties (small-integer and half-integer scores), also K = 1 and K = n."""
    say(f"topk radix n={n} K={K}")
    d = 128
    q = np.zeros((1, 2, 3, d), np.float32)
    q[..., 0] = 1.0
    q[0, :, 1, 1] = -0.5
    q[0, :, 2, 0] = -1.0
    rng = np.random.default_rng(n + K)
    k = np.zeros((1, 2, n + 3, d), np.float32)
    k[..., 0] = rng.integers(-20, 21, size=(1, 2, n + 3))
    k[..., 1] = rng.integers(-4, 5, size=(1, 2, n + 3))
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda()
    idx, sc = ca.block_score_topk(qt, kt, K, cand_begin=2, cand_count=n, return_scores=True)
    torch.cuda.synchronize()
    ref = orc.block_score_topk(q, k, 2, n, K)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(sc.cpu().numpy(), ref["score"])


def test_topk_random_and_index_build():
    say("topk random + build_kv_index")
    rng = np.random.default_rng(1)
    qm = rng.standard_normal((1, 4, 75, 128)).astype(np.float32) / 8
    km = rng.standard_normal((1, 4, 525, 128)).astype(np.float32) / 8
    cm = qm.mean(axis=2, keepdims=True).astype(np.float32)
    qt, kt, ct = (torch.from_numpy(x).cuda() for x in (qm, km, cm))
    pers = ca.block_score_topk(ct, kt, 32, cand_begin=25, cand_count=425)
    loc = ca.block_score_topk(qt, kt, 10, cand_begin=450, cand_count=75)
    torch.cuda.synchronize()
    rp = orc.block_score_topk(cm, km, 25, 425, 32)
    rl = orc.block_score_topk(qm, km, 450, 75, 10)
    ties = compare_topk(pers, rp) + compare_topk(loc, rl)
    say(f"top-K rows differing at near-ties: {ties}")
    indptr, indices = ca.build_kv_index(1, 4, 75, 0, 25, pers[:, :, 0, :].contiguous(), loc, 0)
    torch.cuda.synchronize()
    ip_ref, ix_ref = orc.build_kv_index(1, 4, 75, 0, 25, pers.cpu().numpy()[:, :, 0, :], loc.cpu().numpy(), 0)
    np.testing.assert_array_equal(indptr.cpu().numpy(), ip_ref)
    np.testing.assert_array_equal(indices.cpu().numpy()[:len(ix_ref)], ix_ref)


def test_build_kv_index_dedup_and_offset():
    say("build_kv_index dedup/offset")
    pers = np.array([[[1, 2, 30], [0, 5, 6]]], np.int32)                    # [1, 2, 3]
    topk = np.array([[[[0, 29]], [[3, 4]]]], np.int32).repeat(2, axis=2)   # [1, 2, 2, 2]
    topk = np.ascontiguousarray(topk.reshape(1, 2, 2, 2))
    ip, ix = ca.build_kv_index(1, 2, 2, 0, 3, i32(pers), i32(topk), 1)
    torch.cuda.synchronize()
    ipr, ixr = orc.build_kv_index(1, 2, 2, 0, 3, pers, topk, 1)
    np.testing.assert_array_equal(ip.cpu().numpy(), ipr)
    np.testing.assert_array_equal(ix.cpu().numpy()[:len(ixr)], ixr)


@pytest.mark.parametrize("cb,cc,K,pb,pc,off", [
    (25, 425, 32, 0, 25, 0),        # shared list: sink prefix + persistent ids (1024 threads)
    (0, 75, 10, 0, 0, 450),         # local list: window-relative ids + offset (256 threads)
    (400, 100, 7, 10, 300, 0),      # prefix longer than the workgroup
    (3, 4, 4, 0, 3, 0),             # K = candidate count
])
def test_topk_lists_match_separate_index_build(cb, cc, K, pb, pc, off):
    """Selection and block lists in one launch equal the separate top-K
    launch followed by the list merge (the oracle's build_kv_index)."""
    say(f"topk lists cb={cb} cc={cc} K={K} prefix={pb}+{pc} off={off}")
    rng = np.random.default_rng(cb + cc + K)
    B, H, NQB = 2, 3, 37
    qm = rng.standard_normal((B, H, NQB, 128)).astype(np.float32) / 8
    km = rng.standard_normal((B, H, cb + cc + 5, 128)).astype(np.float32) / 8
    qt, kt = torch.from_numpy(qm).cuda(), torch.from_numpy(km).cuda()
    idx, ip, ix = ca.block_score_topk_lists(qt, kt, K, cand_begin=cb, cand_count=cc,
                                            prefix_begin=pb, prefix_count=pc, id_offset=off)
    ref_idx = ca.block_score_topk(qt, kt, K, cand_begin=cb, cand_count=cc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx.cpu().numpy())
    ipr, ixr = orc.build_kv_index(B, H, NQB, pb, pc, None, idx.cpu().numpy(), off)
    np.testing.assert_array_equal(ip.cpu().numpy(), ipr)
    np.testing.assert_array_equal(ix.cpu().numpy(), ixr)


def test_topk_batch_equals_separate_calls():
    """Selections of different shapes in one launch (the block-sparse path's
    persistent and local pair, a plain top-K, a 4096-candidate radix case):
    ids and block lists bit for bit as the separate calls, ids against the
    oracle."""
    say("topk batch")
    rng = np.random.default_rng(3)
    t = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32) / 8).cuda()
    cm, km = t(1, 12, 1, 128), t(1, 12, 525, 128)
    qm, kl = t(1, 12, 75, 128), t(1, 12, 75, 128)
    q3, k3 = t(2, 3, 7, 64), t(2, 3, 300, 64)
    q4, k4 = t(1, 2, 2, 128), t(1, 2, 4100, 128)
    jobs = [dict(q_mean=cm, k_mean=km, K=32, cand_begin=25, cand_count=425, prefix_begin=0,
                 prefix_count=25, lists=True),
            dict(q_mean=qm, k_mean=kl, K=10, cand_begin=0, cand_count=75, id_offset=450, lists=True),
            dict(q_mean=q3, k_mean=k3, K=17, cand_begin=20, cand_count=250),
            dict(q_mean=q4, k_mean=k4, K=300, cand_begin=4, cand_count=4096)]
    (p1, ip1, ix1), (p2, ip2, ix2), p3, p4 = ca.block_score_topk_batch(jobs)
    s1 = ca.block_score_topk_lists(cm, km, 32, cand_begin=25, cand_count=425, prefix_begin=0, prefix_count=25)
    s2 = ca.block_score_topk_lists(qm, kl, 10, cand_begin=0, cand_count=75, id_offset=450)
    s3 = ca.block_score_topk(q3, k3, 17, cand_begin=20, cand_count=250)
    s4 = ca.block_score_topk(q4, k4, 300, cand_begin=4, cand_count=4096)
    torch.cuda.synchronize()
    for a, b in [(p1, s1[0]), (ip1, s1[1]), (ix1, s1[2]), (p2, s2[0]), (ip2, s2[1]), (ix2, s2[2]),
                 (p3, s3), (p4, s4)]:
        assert torch.equal(a, b)
    for idx, (qq, kk, cb, cc, K) in [(p1, (cm, km, 25, 425, 32)), (p3, (q3, k3, 20, 250, 17)),
                                     (p4, (q4, k4, 4, 4096, 300))]:
        compare_topk(idx, orc.block_score_topk(qq.cpu().numpy(), kk.cpu().numpy(), cb, cc, K))


@pytest.mark.parametrize("d", [64, 128])
def test_block_mean_pair_equals_two_calls(d):
    """Two tensors in one launch (the second a window of a longer cache, so
    with its own strides): each output bit for bit as its own ca_block_mean
    call, and against the oracle."""
    say(f"block_mean pair d={d}")
    X = _gen(61, 1, 1560 * 2 + 100, 3, d, 2.0)
    Y = _gen(62, 1, 1560 * 5, 3, d, 1.0)
    x, y = to_dev(X), to_dev(Y)
    yw = y[:, 1560 * 2:1560 * 2 + x.shape[1]]
    m1, m2, tot = ca.block_mean_pair(x, yw, 64, 1560, with_total=True)
    r1, rt = ca.block_mean(x, 64, 1560, with_total=True)
    r2 = ca.block_mean(yw, 64, 1560)
    torch.cuda.synchronize()
    assert torch.equal(m1, r1) and torch.equal(m2, r2) and torch.equal(tot, rt)
    np.testing.assert_allclose(m2.cpu().numpy(), orc.block_mean(Y.f32[:, 1560 * 2:1560 * 2 + X.f32.shape[1]],
                                                                64, 1560), rtol=0, atol=2e-6)


@pytest.mark.parametrize("d", [24, 64, 128, 512])
def test_block_mean_with_chunk_mean(d):
    """Block means and the mean over all tokens (the chunk-mean query), for
    head dims below, at and above one thread per column of the reduction."""
    say(f"block_mean + chunk mean d={d}")
    X = _gen(51, 1, 1560 * 2 + 100, 3, d, 2.0)
    m, tot = ca.block_mean(to_dev(X), 64, 1560, with_total=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().numpy(), orc.block_mean(X.f32, 64, 1560), rtol=0, atol=2e-6)
    np.testing.assert_allclose(tot.cpu().numpy(), orc.chunk_mean_query(X.f32), rtol=0, atol=2e-6)


@pytest.mark.parametrize("d", [4, 12, 64, 96, 256, 512])
def test_topk_head_dims(d):
    """Cooperative (d/4 a power of two up to 64) and per-thread scoring paths."""
    say(f"topk d={d}")
    rng = np.random.default_rng(d)
    qm = rng.standard_normal((1, 3, 7, d)).astype(np.float32)
    km = rng.standard_normal((1, 3, 300, d)).astype(np.float32)
    qt, kt = torch.from_numpy(qm).cuda(), torch.from_numpy(km).cuda()
    for K, cb, cc in [(10, 20, 75), (32, 0, 300), (1, 299, 1)]:
        idx, sc = ca.block_score_topk(qt, kt, K, cand_begin=cb, cand_count=cc, return_scores=True)
        torch.cuda.synchronize()
        ref = orc.block_score_topk(qm, km, cb, cc, K)
        compare_topk(idx, ref)
        same = np.all(idx.cpu().numpy() == ref["idx"], axis=-1)
        np.testing.assert_allclose(sc.cpu().numpy()[same], ref["score"][same], rtol=1e-5, atol=1e-5 * d)


@pytest.mark.parametrize("NQB", [3, 200])
def test_build_kv_index_overlapping_lists(NQB):
    """Sink, persistent and top-K lists that overlap and repeat ids, on few
    long rows (one thread per output id) and many rows (one thread per row)."""
    say(f"build_kv_index overlaps NQB={NQB}")
    rng = np.random.default_rng(NQB)
    B, H, C, K = 1, 2, 12, 9
    pers = np.sort(rng.choice(40, size=(B, H, C), replace=True), axis=-1).astype(np.int32)
    topk = np.sort(rng.choice(30, size=(B, H, NQB, K), replace=True), axis=-1).astype(np.int32)
    ip, ix = ca.build_kv_index(B, H, NQB, 4, 10, i32(pers), i32(topk), 7)
    torch.cuda.synchronize()
    ipr, ixr = orc.build_kv_index(B, H, NQB, 4, 10, pers, topk, 7)
    np.testing.assert_array_equal(ip.cpu().numpy(), ipr)
    np.testing.assert_array_equal(ix.cpu().numpy()[:len(ixr)], ixr)


def test_build_kv_index_unstaged_large():
    """More persistent + top-K ids than the LDS staging holds: the merges read
    global memory directly."""
    say("build_kv_index large")
    rng = np.random.default_rng(7)
    B, H, NQB, C, K = 1, 8, 300, 16, 8
    pers = np.sort(rng.choice(200, size=(B, H, C), replace=True), axis=-1).astype(np.int32)
    topk = np.sort(rng.choice(60, size=(B, H, NQB, K), replace=True), axis=-1).astype(np.int32)
    ip, ix = ca.build_kv_index(B, H, NQB, 5, 20, i32(pers), i32(topk), 150)
    torch.cuda.synchronize()
    ipr, ixr = orc.build_kv_index(B, H, NQB, 5, 20, pers, topk, 150)
    np.testing.assert_array_equal(ip.cpu().numpy(), ipr)
    np.testing.assert_array_equal(ix.cpu().numpy()[:len(ixr)], ixr)


# ---------------------------------------------------------------------------
# workload-sized cases, exactly as the benchmark runs them.  Outputs start as
# NaN sentinels, which every element must have overwritten; the whole dense
# layer is compared with the oracle, the other modes on a row in every 32-row
# wave slice of every workgroup, for every head.
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def wan():
    return wl.wan_dense(seed=0)


@pytest.fixture(scope="module")
def wan_dev(wan):
    return to_dev(wan.q), to_dev(wan.k), to_dev(wan.v)


@pytest.fixture(scope="module")
def wan_dense_ref(wan):
    say("oracle: the whole wan dense layer (12 heads x 4680 rows x 32760 keys)")
    return orc.chunk_attn_dense(wan.q.f32, wan.k.f32, wan.v.f32, wan.scale)


@pytest.mark.parametrize("policy", ["auto", "never", "always"])
def test_wan_dense_full_size(wan, wan_dev, wan_dense_ref, policy):
    # auto: the schedule bench.py times; never: the plain grid, one workgroup
    # per (head, 256-query tile); always: the balanced schedule
    say(f"wan dense 12x4680x32760 d128, split policy {policy}, whole layer")
    q, k, v = wan_dev
    o, l = nan_out(1, wan.Nq, wan.H, wan.d), nan_lse(1, wan.H, wan.Nq)
    ca.chunk_attn_fwd(q, k, v, scale=wan.scale, balanced=policy, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("wan dense", o, l)
    Or, Lr = wan_dense_ref
    assert_o(o, Or, True, f"wan dense {policy}")
    assert_lse(l, Lr, f"wan dense {policy}")


def test_wan_local_history_merge_full_size(wan, wan_dev, wan_dense_ref):
    say("wan local/history merge, whole layer")
    q, k, v = wan_dev
    outs = []
    for key in ("local_blocks", "history_blocks"):
        blocks = np.array(wan.meta[key], np.int32)
        ip = np.arange(wan.H + 1, dtype=np.int32) * len(blocks)
        ix = np.tile(blocks, wan.H)
        ob = nan_out(1, wan.Nq, wan.H, wan.d, torch.float32)
        lb = nan_lse(1, wan.H, wan.Nq)
        ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip), kv_indices=i32(ix), kv_block=64,
                          kv_seg=1560, q_block=wan.Nq, q_seg=wan.Nq, scale=wan.scale,
                          out=ob, lse=lb)
        outs.append((ob, lb))
    om, lm = nan_out(1, wan.Nq, wan.H, wan.d), nan_lse(1, wan.H, wan.Nq)
    ca.lse_merge(outs[0][0], outs[0][1], outs[1][0], outs[1][1], out=om, out_lse=lm)
    torch.cuda.synchronize()
    assert_written("wan merge branches", outs[0][0], outs[0][1], outs[1][0], outs[1][1])
    assert_written("wan merge", om, lm)
    Or, Lr = wan_dense_ref
    assert_o(om, Or, True, "wan merge")
    assert_lse(lm, Lr, "wan merge")


def _union_csr(info, H, nqb):
    """Per (h, qb) row: the head's shared list followed by the row's local list."""
    sp, sx = info["shared_indptr"].cpu().numpy(), info["shared_indices"].cpu().numpy()
    lp, lx = info["local_indptr"].cpu().numpy(), info["local_indices"].cpu().numpy()
    rows = []
    for h in range(H):
        for qb in range(nqb):
            r = h * nqb + qb
            rows.append(np.concatenate([sx[sp[h]:sp[h + 1]], lx[lp[r]:lp[r + 1]]]))
    ip = np.zeros(len(rows) + 1, np.int32)
    ip[1:] = np.cumsum([len(x) for x in rows])
    return ip, np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("ratio", [0.25, 0.125, 0.0625])
def test_wan_block_sparse_pipeline(wan, wan_dev, ratio):
    say(f"wan block-sparse ratio={ratio}")
    q, k, v = wan_dev
    lay = wl.sparse_layout(wan, ratio)
    o, l = nan_out(1, wan.Nq, wan.H, wan.d), nan_lse(1, wan.H, wan.Nq)
    _, _, info = ca.block_sparse_fwd(q, k, v, sink_begin=0, sink_count=lay["sink_count"],
                                     hist_begin=lay["hist_begin"], hist_count=lay["hist_count"],
                                     C=lay["C"], local_begin=lay["local_begin"],
                                     local_count=lay["local_count"], K=lay["K"], block=64,
                                     seg=1560, scale=wan.scale, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("wan sparse", o, l)
    sel = orc.sparse_selection(wan.q.f32, wan.k.f32, 64, 1560, 64, 1560, lay)
    np.testing.assert_allclose(info["q_mean"].cpu().numpy(), sel["q_mean"], rtol=0, atol=5e-6)
    np.testing.assert_allclose(info["k_mean"].cpu().numpy(), sel["k_mean"], rtol=0, atol=5e-6)
    np.testing.assert_allclose(info["chunk_mean"].cpu().numpy(), sel["chunk_mean"], rtol=0, atol=5e-6)
    ties = (compare_topk(info["persistent"], sel["persistent"], what="persistent")
            + compare_topk(info["local"] + info["local_base"], sel["local"], what="local"))
    say(f"top-K rows differing at near-ties: {ties}")
    ip, ix = _union_csr(info, wan.H, 75)
    if ties == 0:
        # the shared + local lists together are exactly the PBSA block list
        for r in range(len(ip) - 1):
            np.testing.assert_array_equal(np.sort(ix[ip[r]:ip[r + 1]]),
                                          sel["indices"][sel["indptr"][r]:sel["indptr"][r + 1]])
    # attention over the selected lists (as built on the GPU, checked above),
    # on a row of every 32-row wave slice of every query block and tile
    rows = wave_rows(wan.Nq, 64, 1560, seed=int(ratio * 1000))
    Or, Lr = orc.chunk_attn_blocks(wan.q.f32, wan.k.f32, wan.v.f32, ip, ix, 64, 1560, 64, 1560,
                                   wan.scale, rows=rows)
    assert_o(o[:, rows], Or, True, f"wan sparse {ratio}")
    assert_lse(l[:, :, rows], Lr, f"wan sparse {ratio}")


@pytest.mark.parametrize("lay", [
    # sink above the history range: the shared list is merged by a separate launch
    dict(sink_begin=8, sink_count=4, hist_begin=0, hist_count=8, C=3, local_begin=12,
         local_count=4, K=2),
    # no persistent blocks
    dict(sink_begin=0, sink_count=2, hist_begin=2, hist_count=10, C=0, local_begin=12,
         local_count=4, K=2),
    # no top-K blocks: the local pass resumes over empty lists
    dict(sink_begin=0, sink_count=1, hist_begin=1, hist_count=11, C=4, local_begin=12,
         local_count=4, K=0),
])
def test_block_sparse_layouts(lay):
    """Layouts off the fused path (the block lists assembled by a separate
    launch, or absent): selection and attention against the oracle."""
    say(f"block-sparse layout {lay}")
    w = wl.tiny_dense(seed=5)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o, l, info = ca.block_sparse_fwd(q, k, v, block=64, seg=256, scale=w.scale, **lay)
    torch.cuda.synchronize()
    nqb = w.Nq // 64
    sel = orc.sparse_selection(w.q.f32, w.k.f32, 64, 256, 64, 256,
                               dict(lay, C=max(lay["C"], 1), K=max(lay["K"], 1)))
    if lay["C"]:
        assert compare_topk(info["persistent"], sel["persistent"]) == 0
    if lay["K"]:
        assert compare_topk(info["local"] + info["local_base"], sel["local"]) == 0
    ip, ix = _union_csr(info, w.B * w.H, nqb)
    pers = sel["persistent"]["idx"][:, :, 0, :] if lay["C"] else np.zeros((w.B, w.H, 0), np.int32)
    loc = sel["local"]["idx"] if lay["K"] else np.zeros((w.B, w.H, nqb, 0), np.int32)
    ipr, ixr = orc.build_kv_index(w.B, w.H, nqb, lay["sink_begin"], lay["sink_count"], pers, loc, 0)
    for r in range(len(ip) - 1):
        np.testing.assert_array_equal(np.sort(ix[ip[r]:ip[r + 1]]), ixr[ipr[r]:ipr[r + 1]])
    Or, Lr = orc.chunk_attn_blocks(w.q.f32, w.k.f32, w.v.f32, ip, ix, 64, 256, 64, 256, w.scale)
    assert_o(o, Or, True, "layout sparse")
    assert_lse(l, Lr, "layout sparse")


def test_wan_block_sparse_resident_key_means(wan, wan_dev):
    """With the history key-block means passed in as resident state, only the
    local window's means are recomputed (over that window alone); the
    selection and the output are identical to computing every mean."""
    say("wan block-sparse with resident key means")
    q, k, v = wan_dev
    lay = wl.sparse_layout(wan, 0.125)
    args = dict(sink_begin=0, sink_count=lay["sink_count"], hist_begin=lay["hist_begin"],
                hist_count=lay["hist_count"], C=lay["C"], local_begin=lay["local_begin"],
                local_count=lay["local_count"], K=lay["K"], block=64, seg=1560, scale=wan.scale)
    o0, l0, i0 = ca.block_sparse_fwd(q, k, v, **args)
    o1, l1, i1 = ca.block_sparse_fwd(q, k, v, k_mean=i0["k_mean"].clone(), **args)
    torch.cuda.synchronize()
    assert i1["local_base"] == lay["local_begin"] and i1["k_mean_local"].shape[2] == lay["local_count"]
    assert torch.equal(i1["k_mean_local"], i0["k_mean"][:, :, lay["local_begin"]:])
    assert torch.equal(i1["local"] + i1["local_base"], i0["local"])
    assert torch.equal(i1["local_indices"], i0["local_indices"])
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


@pytest.mark.parametrize("q_block,alias", [(64, False), (256, False), (256, True)])
def test_resume_from_branch_equals_union(q_block, alias):
    say(f"resume q_block={q_block} alias={alias}")
    w = wl.tiny_dense(seed=4)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    nqb = w.Nq // q_block
    rows = w.B * w.H * nqb
    loc, hist = w.meta["local_blocks"], w.meta["history_blocks"]
    ip1 = np.arange(w.B * w.H + 1, dtype=np.int32) * len(hist)
    o1, l1 = ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip1), kv_indices=i32(np.tile(hist, w.B * w.H)),
                               kv_block=64, kv_seg=w.Nkv, q_block=w.Nq, q_seg=w.Nq,
                               out_dtype=torch.float32)
    ip2 = np.arange(rows + 1, dtype=np.int32) * len(loc)
    kw = dict(out=o1, lse=l1) if alias else dict(out_dtype=torch.bfloat16)
    o, l = ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip2), kv_indices=i32(np.tile(loc, rows)),
                             kv_block=64, kv_seg=w.Nkv, q_block=q_block, q_seg=w.Nq,
                             o_init=o1, lse_init=l1, **kw)
    torch.cuda.synchronize()
    Od, Ld = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale)
    assert_o(o, Od, not alias, "resumed vs dense")
    assert_lse(l, Ld, "resumed vs dense")


def test_resume_from_empty_branch_and_into_empty_set():
    say("resume edge cases")
    B, H, Nq, Nkv, d = 1, 2, 100, 130, 128
    Q, K, V = _gen(60, B, Nq, H, d), _gen(61, B, Nkv, H, d), _gen(62, B, Nkv, H, d)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    zero_o = torch.zeros((B, Nq, H, d), dtype=torch.float32, device="cuda")
    ninf = torch.full((B, H, Nq), float("-inf"), device="cuda")
    o, l = ca.chunk_attn_fwd(q, k, v, o_init=zero_o, lse_init=ninf, out_dtype=torch.float32)
    Od, Ld = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert_o(o, Od, False, "resume from empty")
    assert_lse(l, Ld, "resume from empty")
    # an empty key set after a branch passes the branch through
    ip = torch.zeros(B * H * 2 + 1, dtype=torch.int32, device="cuda")
    o2, l2 = ca.chunk_attn_fwd(q, k, v, kv_indptr=ip, kv_indices=ip, q_block=64, q_seg=Nq,
                               o_init=o, lse_init=l, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.allclose(o2, o, atol=1e-6, rtol=0) and torch.allclose(l2, l, atol=1e-6, rtol=0)


def test_ragged_full_size():
    say("ragged 12 heads, cu_seqlens")
    w = wl.ragged(seed=0)
    o, l = nan_out(1, w.Nq, w.H, w.d), nan_lse(1, w.H, w.Nq)
    ca.chunk_attn_varlen_fwd(to_dev(w.q), to_dev(w.k_flat), to_dev(w.v_flat), i32(w.cu_seqlens),
                             cu_seqlens_host=w.cu_seqlens, scale=w.scale, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("ragged", o, l)
    rows = wave_rows(w.Nq, seed=3)
    Or, Lr = orc.chunk_attn_varlen(w.q.f32, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens, w.scale, rows=rows)
    assert_o(o[:, rows], Or, True, "ragged")
    assert_lse(l[:, :, rows], Lr, "ragged")


@pytest.mark.parametrize("pbsa", [False, True])
def test_mixed_40_heads_full_size(pbsa):
    say(f"mixed 40 heads, block-list heads as {'one-pass PBSA' if pbsa else 'union lists'}")
    w = wl.mixed(seed=0)
    lay = w.meta["sparse"]
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    sparse_heads = [h for h in range(w.H) if w.head_mode[h] == 1]
    # selection for the block-sparse heads runs on the GPU over those heads' views
    hsel = torch.tensor(sparse_heads, device="cuda")
    qs, ks = q.index_select(2, hsel).contiguous(), k.index_select(2, hsel).contiguous()
    qm, km, cm = ca.block_mean(qs, 64, 1560), ca.block_mean(ks, 64, 1560), ca.block_mean(qs, w.Nq, w.Nq)
    pers = ca.block_score_topk(cm, km, lay["C"], cand_begin=lay["hist_begin"], cand_count=lay["hist_count"])
    loc = ca.block_score_topk(qm, km, lay["K"], cand_begin=lay["local_begin"], cand_count=lay["local_count"])
    ip_s, ix_s = ca.build_kv_index(1, len(sparse_heads), 75, 0, lay["sink_count"],
                                   pers[:, :, 0, :].contiguous(), loc, 0)
    torch.cuda.synchronize()
    # scatter the per-sparse-head rows into a CSR over all 40 heads (other heads empty)
    ip_s, ix_s = ip_s.cpu().numpy(), ix_s.cpu().numpy()
    lists = []
    for h in range(w.H):
        for qb in range(75):
            if w.head_mode[h] == 1:
                r = sparse_heads.index(h) * 75 + qb
                lists.append(ix_s[ip_s[r]:ip_s[r + 1]])
            else:
                lists.append(np.zeros(0, np.int32))
    ip = np.zeros(len(lists) + 1, np.int32)
    ip[1:] = np.cumsum([len(x) for x in lists])
    ix = np.concatenate(lists).astype(np.int32)
    extra = {}
    if pbsa:
        # the same key sets split as PBSA takes them: per head the sink and
        # persistent blocks, per query block its top-K window blocks
        pn, ln = pers.cpu().numpy(), loc.cpu().numpy()
        sink = np.arange(lay["sink_count"], dtype=np.int32)
        shared, local = [], []
        for h in range(w.H):
            si = sparse_heads.index(h) if w.head_mode[h] == 1 else -1
            shared.append(np.concatenate([sink, pn[0, si, 0]]) if si >= 0 else np.zeros(0, np.int32))
            for qb in range(75):
                local.append(ln[0, si, qb] if si >= 0 else np.zeros(0, np.int32))
        sp = np.zeros(w.H + 1, np.int32)
        sp[1:] = np.cumsum([len(x) for x in shared])
        lp = np.zeros(len(local) + 1, np.int32)
        lp[1:] = np.cumsum([len(x) for x in local])
        extra = dict(kv_shared_indptr=i32(sp), kv_shared_indices=i32(np.concatenate(shared)))
        call_ip, call_ix = i32(lp), i32(np.concatenate(local))
    else:
        call_ip, call_ix = i32(ip), i32(ix)
    o, l = nan_out(1, w.Nq, w.H, w.d), nan_lse(1, w.H, w.Nq)
    ca.chunk_attn_mixed_fwd(q, w.head_mode, k=k, v=v, kv_indptr=call_ip, kv_indices=call_ix,
                            kv_block=64, kv_seg=1560, q_block=64, q_seg=1560, **extra,
                            k_flat=to_dev(w.k_flat), v_flat=to_dev(w.v_flat),
                            cu_seqlens=i32(w.cu_seqlens), cu_seqlens_host=w.cu_seqlens,
                            scale=w.scale, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("mixed", o, l)
    rows = wave_rows(w.Nq, 64, 1560, seed=4)
    og, lg = o[:, rows].float().cpu().numpy(), l[:, :, rows].cpu().numpy()
    for mode in range(3):
        hs = [h for h in range(w.H) if w.head_mode[h] == mode]
        if mode == 0:
            Or, Lr = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale, rows=rows, heads=hs)
        elif mode == 1:
            Or, Lr = orc.chunk_attn_blocks(w.q.f32, w.k.f32, w.v.f32, ip, ix, 64, 1560, 64, 1560,
                                           w.scale, rows=rows, heads=hs)
        else:
            Or, Lr = orc.chunk_attn_varlen(w.q.f32, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens,
                                           w.scale, rows=rows, heads=hs)
        assert_o(torch.from_numpy(og[:, :, hs]), Or, True, f"mixed mode {mode}")
        assert_lse(torch.from_numpy(lg[:, hs]), Lr, f"mixed mode {mode}")

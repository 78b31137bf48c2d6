"""Pins of the CPU oracle to facts outside itself (CPU only).

Each check compares the oracle with something it does not compute the same
way: the literal definition in pure-Python loops, closed forms, scipy
routines the oracle never calls, identities stated on the pages (the LSE
merge of disjoint branches equals attention over their union), cross-mode
identities (all blocks = dense, ragged = gathered frames) and planted
orderings for the top-K.  The planted-mistake tests at the end show that a
plausible slip in the oracle makes one of these pins fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import special

import oracle
from oracle import chunk_attention as oc
from kv_cache_attention_chunk_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def brute_attention(q, k, v, scale):
    """The definition, term by term, in Python floats with math.fsum."""
    n, m = len(q), len(k)
    O, L = [], []
    for i in range(n):
        e = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j])))
             for j in range(m)]
        z = math.fsum(e)
        O.append([math.fsum(e[j] * float(v[j][c]) for j in range(m)) / z
                  for c in range(len(v[0]))])
        L.append(math.log(z))
    return np.array(O), np.array(L)


def check_attention_bruteforce(attn):
    rng = np.random.default_rng(11)
    for n, m, d in [(1, 1, 4), (3, 7, 8), (5, 13, 16), (8, 48, 16), (2, 33, 5)]:
        q, k, v = _rand(rng, n, d), _rand(rng, m, d), _rand(rng, m, d + 3)
        scale = 1.0 / math.sqrt(d)
        o, l = attn(q, k, v, scale)
        bo, bl = brute_attention(q, k, v, scale)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, bl, rtol=0, atol=1e-12)


def test_attention_matches_bruteforce_definition():
    check_attention_bruteforce(oc.attention)


def check_attention_closed_forms(attn):
    rng = np.random.default_rng(5)
    d, m = 16, 37
    k, v = _rand(rng, m, d), _rand(rng, m, d)
    # q = 0: uniform weights -> O = mean(V), LSE = ln m
    o, l = attn(np.zeros((2, d), np.float32), k, v, 0.25)
    np.testing.assert_allclose(o, np.tile(v.astype(np.float64).mean(0), (2, 1)), atol=1e-13)
    np.testing.assert_allclose(l, [math.log(m)] * 2, atol=1e-13)
    # a single key: O = v, LSE = its scaled logit
    q = _rand(rng, 3, d)
    o, l = attn(q, k[:1], v[:1], 0.3)
    np.testing.assert_allclose(o, np.tile(v[:1].astype(np.float64), (3, 1)), atol=1e-13)
    np.testing.assert_allclose(l, 0.3 * (q.astype(np.float64) @ k[0].astype(np.float64)), atol=1e-12)
    # every key/value duplicated: O unchanged, LSE + ln 2
    o1, l1 = attn(q, k, v, 0.3)
    o2, l2 = attn(q, np.concatenate([k, k]), np.concatenate([v, v]), 0.3)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + math.log(2.0), atol=1e-12)
    # constant V rows: O equals that row whatever the weights
    vc = np.tile(_rand(rng, 1, d), (m, 1))
    o, _ = attn(q, k, vc, 0.3)
    np.testing.assert_allclose(o, np.tile(vc[:1].astype(np.float64), (3, 1)), atol=1e-12)
    # permuting the key set changes nothing
    perm = rng.permutation(m)
    o3, l3 = attn(q, k[perm], v[perm], 0.3)
    np.testing.assert_allclose(o3, o1, atol=1e-12)
    np.testing.assert_allclose(l3, l1, atol=1e-12)
    # one key far above the others: O -> its value row
    kd = k.copy()
    kd[7] = 40.0 * q[0] / np.linalg.norm(q[0])
    o, _ = attn(q[:1], kd, v, 1.0)
    np.testing.assert_allclose(o[0], v[7], atol=1e-9)
    # large logits (no overflow): LSE = max logit + ln(count of maxima)
    o, l = attn(np.full((1, d), 30.0, np.float32), np.full((4, d), 30.0, np.float32), v[:4], 1.0)
    np.testing.assert_allclose(l, [30.0 * 30.0 * d + math.log(4)], rtol=1e-15)
    np.testing.assert_allclose(o[0], v[:4].astype(np.float64).mean(0), atol=1e-12)
    # empty key set
    o, l = attn(q, k[:0], v[:0], 0.3)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_attention_closed_forms():
    check_attention_closed_forms(oc.attention)


def test_attention_matches_scipy():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 9, 32), _rand(rng, 200, 32), _rand(rng, 200, 32)
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * 0.177
    o, l = oc.attention(q, k, v, 0.177)
    np.testing.assert_allclose(l, special.logsumexp(s, axis=1), atol=1e-12)
    np.testing.assert_allclose(o, special.softmax(s, axis=1) @ v.astype(np.float64), atol=1e-12)


def test_dense_layout_and_sampled_rows():
    rng = np.random.default_rng(4)
    B, Nq, Nkv, H, d = 2, 6, 20, 3, 8
    Q, K, V = _rand(rng, B, Nq, H, d), _rand(rng, B, Nkv, H, d), _rand(rng, B, Nkv, H, d)
    O, L = oc.chunk_attn_dense(Q, K, V, 0.5)
    assert O.shape == (B, Nq, H, d) and L.shape == (B, H, Nq)
    for b, h, i in itertools.product(range(B), range(H), range(Nq)):
        bo, bl = brute_attention(Q[b, i:i + 1, h], K[b, :, h], V[b, :, h], 0.5)
        np.testing.assert_allclose(O[b, i, h], bo[0], atol=1e-12)
        np.testing.assert_allclose(L[b, h, i], bl[0], atol=1e-12)
    Os, Ls = oc.chunk_attn_dense(Q, K, V, 0.5, rows=[5, 0, 3], heads=[2, 0])
    np.testing.assert_array_equal(Os, O[:, [5, 0, 3]][:, :, [2, 0]])
    np.testing.assert_array_equal(Ls, L[:, [2, 0]][:, :, [5, 0, 3]])


# --------------------------------------------------------------------------
# LSE merge: the pages' identity -- local and history branches recombined
# through their LSE equal attention over the union.
# --------------------------------------------------------------------------
def check_merge_identity(merge, attn):
    rng = np.random.default_rng(7)
    n, m, d = 5, 61, 16
    q, k, v = _rand(rng, n, d), 2 * _rand(rng, m, d), _rand(rng, m, d)
    for split in [rng.permutation(m)[:20], np.arange(0, m, 3), np.array([4])]:
        a = np.zeros(m, bool)
        a[split] = True
        o1, l1 = attn(q, k[a], v[a], 0.25)
        o2, l2 = attn(q, k[~a], v[~a], 0.25)
        o, l = merge(o1, l1, o2, l2)
        of, lf = attn(q, k, v, 0.25)
        np.testing.assert_allclose(o, of, atol=1e-12)
        np.testing.assert_allclose(l, lf, atol=1e-12)


def test_merge_equals_attention_over_union():
    check_merge_identity(oc.lse_merge, oc.attention)


def test_merge_special_cases():
    rng = np.random.default_rng(8)
    o1, o2 = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    l1 = rng.standard_normal(4)
    # equal LSE: plain average, LSE + ln 2
    o, l = oc.lse_merge(o1, l1, o2, l1)
    np.testing.assert_allclose(o, (o1 + o2) / 2, atol=1e-14)
    np.testing.assert_allclose(l, l1 + math.log(2), atol=1e-14)
    # an empty branch (-inf) passes the other through
    o, l = oc.lse_merge(o1, l1, np.zeros_like(o2), np.full(4, -np.inf))
    np.testing.assert_allclose(o, o1, atol=0)
    np.testing.assert_allclose(l, l1, atol=0)
    o, l = oc.lse_merge(np.zeros_like(o1), np.full(4, -np.inf), o2, l1)
    np.testing.assert_allclose(o, o2, atol=0)
    # both empty
    o, l = oc.lse_merge(o1, np.full(4, -np.inf), o2, np.full(4, -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)
    # very different magnitudes: no overflow
    o, l = oc.lse_merge(o1, np.full(4, 800.0), o2, np.full(4, -800.0))
    np.testing.assert_allclose(o, o1, atol=1e-14)
    np.testing.assert_allclose(l, 800.0, atol=1e-12)


def test_merge_bshd_layout():
    rng = np.random.default_rng(9)
    B, N, H, d = 2, 5, 3, 4
    O1, O2 = rng.standard_normal((B, N, H, d)), rng.standard_normal((B, N, H, d))
    L1, L2 = rng.standard_normal((B, H, N)), rng.standard_normal((B, H, N))
    O, L = oc.lse_merge_bshd(O1, L1, O2, L2)
    for b, n, h in itertools.product(range(B), range(N), range(H)):
        w1, w2 = math.exp(L1[b, h, n]), math.exp(L2[b, h, n])
        np.testing.assert_allclose(O[b, n, h], (w1 * O1[b, n, h] + w2 * O2[b, n, h]) / (w1 + w2), atol=1e-13)
        np.testing.assert_allclose(L[b, h, n], math.log(w1 + w2), atol=1e-13)


# --------------------------------------------------------------------------
# block tiling, block mode, ragged mode
# --------------------------------------------------------------------------
def test_block_spans_frame_aligned():
    sp = oc.block_spans(1560, 64, 1560)
    assert len(sp) == 25
    assert [tuple(x) for x in sp[:2]] == [(0, 64), (64, 64)]
    assert tuple(sp[24]) == (1536, 24)
    sp = oc.block_spans(21 * 1560, 64, 1560)
    assert len(sp) == 525
    assert tuple(sp[25]) == (1560, 64) and tuple(sp[49]) == (1560 + 1536, 24)
    assert tuple(sp[450]) == (18 * 1560, 64) and tuple(sp[524]) == (20 * 1560 + 1536, 24)
    assert sp[:, 1].sum() == 21 * 1560
    flat = oc.block_spans(1024, 64, 1024)
    assert len(flat) == 16 and np.all(flat[:, 1] == 64) and np.all(flat[:, 0] == 64 * np.arange(16))
    ragged_end = oc.block_spans(100, 64, 60)      # segments 60 + 40
    assert [tuple(x) for x in ragged_end] == [(0, 60), (60, 40)]
    assert [tuple(x) for x in oc.block_spans(150, 64, 150)] == [(0, 64), (64, 64), (128, 22)]


def test_all_blocks_equals_dense_and_sink_plus_recent_equals_gather():
    rng = np.random.default_rng(12)
    B, H, d, seg, blk = 1, 2, 16, 100, 32        # blocks 32,32,32,4 per segment
    Nq, Nkv = 200, 300
    Q, K, V = _rand(rng, B, Nq, H, d), _rand(rng, B, Nkv, H, d), _rand(rng, B, Nkv, H, d)
    nkb = len(oc.block_spans(Nkv, blk, seg))
    nqb = len(oc.block_spans(Nq, blk, seg))
    rows = B * H * nqb
    indptr = np.arange(rows + 1, dtype=np.int32) * nkb
    indices = np.tile(np.arange(nkb, dtype=np.int32), rows)
    O, L = oc.chunk_attn_blocks(Q, K, V, indptr, indices, blk, seg, blk, seg, 0.25)
    Od, Ld = oc.chunk_attn_dense(Q, K, V, 0.25)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(L, Ld, atol=1e-12)
    # a list holding the first segment's blocks = dense attention over tokens 0..99
    first = np.arange(4, dtype=np.int32)
    indices = np.tile(first, rows)
    indptr = np.arange(rows + 1, dtype=np.int32) * 4
    O, L = oc.chunk_attn_blocks(Q, K, V, indptr, indices, blk, seg, blk, seg, 0.25)
    Od, Ld = oc.chunk_attn_dense(Q, K[:, :100], V[:, :100], 0.25)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(L, Ld, atol=1e-12)


def test_block_rows_use_their_own_list():
    rng = np.random.default_rng(13)
    B, H, d, Nq, Nkv, blk = 1, 1, 8, 64, 128, 16
    Q, K, V = _rand(rng, B, Nq, H, d), _rand(rng, B, Nkv, H, d), _rand(rng, B, Nkv, H, d)
    lists = [[0], [7, 2], [], [1, 3, 5]]
    indptr = np.array([0, 1, 3, 3, 6], dtype=np.int32)
    indices = np.array([0, 7, 2, 1, 3, 5], dtype=np.int32)
    O, L = oc.chunk_attn_blocks(Q, K, V, indptr, indices, blk, Nkv, blk, Nq, 0.3)
    for qb, ids in enumerate(lists):
        tok = [t for i in ids for t in range(16 * i, 16 * i + 16)]
        for i in range(16 * qb, 16 * qb + 16):
            if not tok:
                assert np.all(O[0, i, 0] == 0) and L[0, 0, i] == -np.inf
                continue
            bo, bl = brute_attention(Q[0, i:i + 1, 0], K[0, tok, 0], V[0, tok, 0], 0.3)
            np.testing.assert_allclose(O[0, i, 0], bo[0], atol=1e-12)
            np.testing.assert_allclose(L[0, 0, i], bl[0], atol=1e-12)


def test_ragged_equals_gathered_frames_and_block_mode():
    w = wl.ragged(seed=3, H=3, d=16, frames_q=1, frames_kv=6, frame_tokens=40)
    Q, K, V = w.q.f32, w.k.f32, w.v.f32
    O, L = oc.chunk_attn_varlen(Q, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens, w.scale)
    nqb = len(oc.block_spans(w.Nq, 64, 40))
    bpf = 1
    for h in range(3):
        fr = w.ragged_frames[h]
        tok = np.concatenate([np.arange(40 * f, 40 * f + 40) for f in fr])
        Od, Ld = oc.chunk_attn_dense(Q[:, :, h:h + 1], K[:, tok, h:h + 1], V[:, tok, h:h + 1], w.scale)
        np.testing.assert_allclose(O[:, :, h:h + 1], Od, atol=1e-12)
        np.testing.assert_allclose(L[:, h:h + 1], Ld, atol=1e-12)
    # the same through block lists over the dense cache (one 40-token block per frame)
    rows = 3 * nqb
    lists = [np.array(w.ragged_frames[r // nqb], dtype=np.int32) * bpf for r in range(rows)]
    indptr = np.zeros(rows + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(x) for x in lists])
    Ob, Lb = oc.chunk_attn_blocks(Q, K, V, indptr, np.concatenate(lists), 64, 40, 64, 40, w.scale)
    np.testing.assert_allclose(Ob, O, atol=1e-12)
    np.testing.assert_allclose(Lb, L, atol=1e-12)


# --------------------------------------------------------------------------
# block means, coarse scores, top-K, block lists
# --------------------------------------------------------------------------
def test_block_mean_closed_forms():
    B, N, H, d = 1, 1560 * 2, 2, 4
    ramp = np.broadcast_to(np.arange(N, dtype=np.float32)[None, :, None, None], (B, N, H, d))
    m = oc.block_mean(ramp, 64, 1560)
    sp = oc.block_spans(N, 64, 1560)
    expect = sp[:, 0] + (sp[:, 1] - 1) / 2.0          # mean of s .. s+l-1
    for h in range(H):
        np.testing.assert_allclose(m[0, h, :, 0], expect, atol=0)
    assert m.shape == (B, H, 50, d)
    const = np.full((1, 100, 1, 3), 1.25, np.float32)
    np.testing.assert_array_equal(oc.block_mean(const, 64, 100), np.full((1, 1, 2, 3), 1.25))
    rng = np.random.default_rng(2)
    x = _rand(rng, 2, 150, 3, 5)
    mm = oc.block_mean(x, 64, 150)
    for b, h, j in itertools.product(range(2), range(3), range(3)):
        s, l = [(0, 64), (64, 64), (128, 22)][j]
        for c in range(5):
            assert mm[b, h, j, c] == pytest.approx(math.fsum(float(t) for t in x[b, s:s + l, h, c]) / l, abs=1e-15)


def brute_topk(scores, cand, K):
    order = sorted(range(len(cand)), key=lambda j: (-scores[j], cand[j]))
    return sorted(int(cand[j]) for j in order[:K])


def test_topk_planted_order_and_ties():
    d = 8
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    sig = np.array([0.5, 3.0, -1.0, 3.0, 2.0, 0.5, 7.0, 2.0, 3.0, -2.0], np.float32)
    k = np.zeros((1, 1, 14, d), np.float32)
    k[0, 0, 4:14, 0] = sig                              # candidates are blocks 4..13
    r = oc.block_score_topk(q, k, 4, 10, 3)
    # best: 7.0 (blk 10), then the three 3.0s at blocks 5, 7, 12 -> lower ids 5, 7 win
    assert r["idx"][0, 0, 0].tolist() == [5, 7, 10]
    assert r["gap"][0, 0, 0] == 0.0 and r["near_tie"][0, 0, 0] == 3
    assert r["score"][0, 0, 0].tolist() == [3.0, 3.0, 7.0]
    assert oc.block_score_topk(q, k, 4, 10, 1)["idx"][0, 0, 0].tolist() == [10]
    assert oc.block_score_topk(q, k, 4, 10, 10)["idx"][0, 0, 0].tolist() == list(range(4, 14))
    r = oc.block_score_topk(q, k, 4, 10, 5)
    assert r["idx"][0, 0, 0].tolist() == [5, 7, 8, 10, 12]   # 2.0 tie at 8 and 11 -> 8
    # only candidates in range are considered
    k2 = k.copy()
    k2[0, 0, 0, 0] = 100.0
    assert oc.block_score_topk(q, k2, 4, 10, 1)["idx"][0, 0, 0].tolist() == [10]


def test_topk_matches_python_sort_random():
    rng = np.random.default_rng(21)
    qm = _rand(rng, 2, 3, 4, 16)
    km = _rand(rng, 2, 3, 90, 16)
    r = oc.block_score_topk(qm, km, 10, 75, 19)
    for b, h, qb in itertools.product(range(2), range(3), range(4)):
        cand = list(range(10, 85))
        sc = [float(np.float32(math.fsum(float(a) * float(c) for a, c in zip(qm[b, h, qb], km[b, h, j]))))
              for j in cand]
        assert r["idx"][b, h, qb].tolist() == brute_topk(sc, cand, 19)


def test_build_kv_index_set_definition():
    rng = np.random.default_rng(22)
    B, H, NQB, C, K = 1, 3, 5, 4, 2
    pers = np.stack([np.sort(rng.choice(np.arange(25, 100), C, replace=False)) for _ in range(B * H)]).reshape(B, H, C)
    topk = rng.integers(0, 10, size=(B, H, NQB, K))
    topk.sort(axis=-1)
    indptr, indices = oc.build_kv_index(B, H, NQB, 0, 25, pers, topk, 450)
    for h, qb in itertools.product(range(H), range(NQB)):
        r = h * NQB + qb
        row = indices[indptr[r]:indptr[r + 1]].tolist()
        expect = sorted(set(range(25)) | set(pers[0, h].tolist()) | {450 + t for t in topk[0, h, qb]})
        assert row == expect
    # overlapping sets are deduplicated
    ip, ix = oc.build_kv_index(1, 1, 1, 0, 3, np.array([[[1, 2, 5]]]), np.array([[[[5, 6]]]]), 0)
    assert ix.tolist() == [0, 1, 2, 5, 6] and ip.tolist() == [0, 5]


def test_sparse_selection_structure_on_small_frames():
    w = wl.wan_dense(seed=1, H=2, d=32, frames_q=2, frames_kv=6, frame_tokens=150)
    lay = wl.sparse_layout(w, 0.25)
    assert lay["sink_count"] == 3 and lay["local_begin"] == 12 and lay["local_count"] == 6
    lay["C"] = 4
    sel = oc.sparse_selection(w.q.f32, w.k.f32, w.q_block, w.q_seg, w.kv_block, w.kv_seg, lay)
    nqb = 6
    assert sel["q_mean"].shape == (1, 2, nqb, 32)
    for h, qb in itertools.product(range(2), range(nqb)):
        r = h * nqb + qb
        row = sel["indices"][sel["indptr"][r]:sel["indptr"][r + 1]]
        assert row.tolist() == sorted(row.tolist())
        assert set(range(3)) <= set(row.tolist())
        hist = [x for x in row if 3 <= x < 12]
        assert hist == sel["persistent"]["idx"][0, h, 0].tolist()
        loc = [x for x in row if x >= 12]
        assert loc == sel["local"]["idx"][0, h, qb].tolist() and len(loc) == lay["K"]


# --------------------------------------------------------------------------
# figures printed on the pages (tests/golden/page_figures.json)
# --------------------------------------------------------------------------
def test_page_figures_pin_workload_shapes():
    g = json.load(open(GOLDEN))
    w = g["wan_heads"]
    assert w["value"] * w["head_dim"] == w["product"] == 1536
    c = g["wan_cache_21_frames_gb"]
    b = wl.kv_cache_bytes(H=12, d=128, tokens=c["frames"] * wl.FRAME_TOKENS, layers=30)
    assert b == 6_038_323_200
    assert abs(b / 1e9 - c["value"]) / c["value"] < c["approx_rel_tol"]
    m = g["videomla_latent_scalars"]
    assert 2 * 12 * 128 == m["dense_per_token"] and m["d_c"] + m["d_rope"] == m["latent_per_token"]
    assert round(100 * (1 - m["latent_per_token"] / m["dense_per_token"]), 1) == m["reduction_pct"]
    lay = wl.sparse_layout(wl.Workload("x", 1, 1, 8, 4680, 32760, None, None, None, 1.0), g["pbsa_topk_ratio_example"]["value"])
    assert lay["K"] == 5 and lay["local_count"] == 75 and lay["hist_count"] == 425
    assert g["ispa_warmup_frames"]["value"] * wl.FRAME_TOKENS < 32760


# --------------------------------------------------------------------------
# planted mistakes: each plausible slip must trip at least one pin above
# --------------------------------------------------------------------------
def _attn_no_scale(q, k, v, scale):
    return oc.attention(q, k, v, 1.0)


def _attn_swapped_kv(q, k, v, scale):
    return oc.attention(q, v[:, :k.shape[1]], k if k.shape[1] == v.shape[1] else v, scale)


def _attn_lse_without_max(q, k, v, scale):
    o, l = oc.attention(q, k, v, scale)
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) if len(k) else None
    return o, (l - s.max(axis=1) if s is not None else l)


def _attn_transposed_v(q, k, v, scale):
    o, l = oc.attention(q, k, v, scale)
    return o[:, ::-1], l


def _merge_unnormalised(o1, l1, o2, l2):
    o, l = oc.lse_merge(o1, l1, o2, l2)
    M = np.maximum(l1, l2)
    return o * (np.exp(l - M))[..., None], l


def _merge_wrong_sign(o1, l1, o2, l2):
    return oc.lse_merge(o1, -np.asarray(l1), o2, -np.asarray(l2))


@pytest.mark.parametrize("bad", [_attn_no_scale, _attn_swapped_kv, _attn_lse_without_max, _attn_transposed_v])
def test_planted_attention_mistakes_are_caught(bad):
    caught = 0
    for check in (check_attention_bruteforce, check_attention_closed_forms):
        try:
            check(bad)
        except AssertionError:
            caught += 1
    assert caught >= 1


@pytest.mark.parametrize("bad", [_merge_unnormalised, _merge_wrong_sign])
def test_planted_merge_mistakes_are_caught(bad):
    with pytest.raises(AssertionError):
        check_merge_identity(bad, oc.attention)


def test_planted_tiling_and_tiebreak_mistakes_are_caught(monkeypatch):
    def flat_tiling(n, block, seg):
        return np.array([(s, min(block, n - s)) for s in range(0, n, block)], dtype=np.int64)
    monkeypatch.setattr(oc, "block_spans", flat_tiling)
    with pytest.raises(AssertionError):
        test_block_spans_frame_aligned()
    monkeypatch.undo()

    real = oc.block_score_topk

    def reversed_ties(q, k, b, c, K, tie_eps=1e-4):
        # same as the real one, but ties resolved toward the higher block id
        qm = np.asarray(q, np.float64)
        km = np.asarray(k, np.float64)
        cand = np.arange(b, b + c)
        s = (km[0, 0, cand] @ qm[0, 0, 0]).astype(np.float32)
        order = np.lexsort((-cand, -s.astype(np.float64)))
        out = real(q, k, b, c, K)
        out["idx"][0, 0, 0] = np.sort(cand[order[:K]])
        return out
    monkeypatch.setattr(oc, "block_score_topk", reversed_ties)
    with pytest.raises(AssertionError):
        test_topk_planted_order_and_ties()


# ---------------------------------------------------------------------------
# persistent-memory update (Sparse Forcing page, section 2 item 1: evicted
# local-window blocks join the persistent set as candidates; the top C by
# coarse score stay)
# ---------------------------------------------------------------------------
def _planted_update_inputs():
    d = 4
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 1] = 2.0                                      # score = 2 * k[..., 1]
    k = np.zeros((1, 1, 20, d), np.float32)
    # persistent blocks 2, 5, 9 with scores 6, 2, 10; evicted window 14..17 with 8, 2, 12, -4
    for blk, s in [(2, 6.0), (5, 2.0), (9, 10.0), (14, 8.0), (15, 2.0), (16, 12.0), (17, -4.0)]:
        k[0, 0, blk, 1] = s / 2.0
    k[0, 0, 0, 1] = 100.0                                # not a candidate
    pers = np.array([[[2, 5, 9]]], np.int32)
    return q, k, pers


def test_persistent_update_planted_scores_and_ties():
    q, k, pers = _planted_update_inputs()
    r = oc.persistent_update(q, k, pers, 14, 4, 3)
    # candidates by score: 16 (12), 9 (10), 14 (8), 2 (6), 5 (2), 15 (2), 17 (-4)
    assert r["idx"][0, 0].tolist() == [9, 14, 16]
    assert r["score"][0, 0].tolist() == [10.0, 8.0, 12.0]
    assert r["gap"][0, 0] == 2.0
    r5 = oc.persistent_update(q, k, pers, 14, 4, 5)
    # the 2.0 tie between persistent block 5 and evicted block 15: lower id 5 stays
    assert r5["idx"][0, 0].tolist() == [2, 5, 9, 14, 16]
    assert r5["gap"][0, 0] == 0.0 and r5["near_tie"][0, 0] == 2
    # C as large as the candidate set keeps everything, then pads with -1
    r8 = oc.persistent_update(q, k, pers, 14, 4, 8)
    assert r8["idx"][0, 0].tolist() == [2, 5, 9, 14, 15, 16, 17, -1]
    assert r8["score"][0, 0, -1] == -np.inf


def test_persistent_update_set_union_rules():
    q, k, pers = _planted_update_inputs()
    # a persistent id inside the evicted range is one candidate, not two;
    # ids outside [0, NB) are dropped
    p2 = np.array([[[9, 16, 25, -3]]], np.int32)
    r = oc.persistent_update(q, k, p2, 14, 4, 6)
    assert r["idx"][0, 0].tolist() == [9, 14, 15, 16, 17, -1]
    # evicted blocks all below the persistent ones: the set is unchanged
    k_low = k.copy()
    k_low[0, 0, 14:18, 1] = -50.0
    assert oc.persistent_update(q, k_low, pers, 14, 4, 3)["idx"][0, 0].tolist() == [2, 5, 9]
    # evicted blocks all above: the set becomes the best evicted blocks
    k_high = k.copy()
    k_high[0, 0, 14:18, 1] = [60.0, 50.0, 70.0, 40.0]
    assert oc.persistent_update(q, k_high, pers, 14, 4, 3)["idx"][0, 0].tolist() == [14, 15, 16]


def test_persistent_update_matches_bruteforce_random():
    rng = np.random.default_rng(31)
    B, H, NB, d, C = 2, 3, 120, 16, 7
    qm = _rand(rng, B, H, 1, d)
    km = _rand(rng, B, H, NB, d)
    pers = np.stack([np.sort(rng.choice(np.arange(0, 80), C, replace=False))
                     for _ in range(B * H)]).reshape(B, H, C).astype(np.int32)
    r = oc.persistent_update(qm, km, pers, 90, 25, C)
    for b, h in itertools.product(range(B), range(H)):
        cand = sorted(set(range(90, 115)) | set(pers[b, h].tolist()))
        sc = [float(np.float32(math.fsum(float(a) * float(c) for a, c in zip(qm[b, h, 0], km[b, h, j]))))
              for j in cand]
        assert r["idx"][b, h].tolist() == brute_topk(sc, cand, C)


def test_planted_persistent_update_mistakes_are_caught(monkeypatch):
    real = oc.persistent_update

    def evicted_only(q, k, pers, eb, ec, C, tie_eps=1e-4):
        # forgets the current persistent blocks as candidates
        return real(q, k, np.full_like(np.asarray(pers), -1), eb, ec, C, tie_eps)
    monkeypatch.setattr(oc, "persistent_update", evicted_only)
    with pytest.raises(AssertionError):
        test_persistent_update_planted_scores_and_ties()
    monkeypatch.undo()

    def lowest_scores(q, k, pers, eb, ec, C, tie_eps=1e-4):
        # keeps the C worst candidates (sign flipped)
        return real(-np.asarray(q), k, pers, eb, ec, C, tie_eps)
    monkeypatch.setattr(oc, "persistent_update", lowest_scores)
    with pytest.raises(AssertionError):
        test_persistent_update_planted_scores_and_ties()


# ---------------------------------------------------------------------------
# ragged cache packing (Pyramid Forcing page, sections 2-3)
# ---------------------------------------------------------------------------
def test_pack_ragged_copies_equal_the_gathered_frames():
    # copies only: the packed buffers equal the generator's own flattening of
    # the same frame subsets (a separate, data-layout-only implementation)
    w = wl.ragged(seed=3, H=4, d=16, frames_q=1, frames_kv=8, frame_tokens=5)
    fr = w.ragged_frames
    ptr = np.zeros(w.B * w.H + 1, np.int64)
    ptr[1:] = np.cumsum([len(fr[bh]) for bh in range(w.B * w.H)])
    src = np.array([[f, -1] for bh in range(w.B * w.H) for f in fr[bh]], np.int32)
    kf, vf, cu = oc.pack_ragged(w.k.bits, w.v.bits, ptr, src, 5)
    assert np.array_equal(kf, w.k_flat.bits) and np.array_equal(vf, w.v_flat.bits)
    assert np.array_equal(cu, w.cu_seqlens)


def test_pack_ragged_merge_values_and_rounding():
    T, d = 2, 4
    k = np.zeros((1, 3 * T, 1, d), np.float32)
    k[0, 0:T, 0] = [1.0, 2.0, -3.0, 1.0]                  # frame 0
    k[0, T:2 * T, 0] = [2.0, 2.0, 3.0, 1.0078125]         # frame 1 (1 + 2^-7 is one bf16 ulp above 1)
    k[0, 2 * T:, 0] = [8.0, -8.0, 0.5, 0.25]              # frame 2
    # second token rows: averages on and off bf16 rounding ties
    k[0, 1, 0] = [1.0, 1.0, 1.0, -1.0]
    k[0, T + 1, 0] = [1.0234375, 1.01171875, 1.0078125, -1.0234375]
    kb = wl.bf16_bits(k)
    ptr = np.array([0, 4])
    src = np.array([[0, 1], [1, -1], [2, 0], [5, -1]])   # merge, copy, merge, out of range
    kf, vf, cu = oc.pack_ragged(kb, kb, ptr, src, T)
    val = wl.bf16_to_f32(kf).reshape(4, T, d)
    assert val[0, 0].tolist() == [1.5, 2.0, 0.0, 1.0]     # (1 + 1 + 2^-7)/2 = 1 + 2^-8: tie -> even (1.0)
    # 1 + 3*2^-8: tie between odd 1 + 2^-7 and even 1 + 2^-6 -> 1 + 2^-6;
    # 1 + 3*2^-9 (above the tie at 1 + 2^-8) -> 1 + 2^-7; 1 + 2^-8 -> 1.0; sign kept
    assert val[0, 1].tolist() == [1.015625, 1.0078125, 1.0, -1.015625]
    assert val[1, 0].tolist() == [2.0, 2.0, 3.0, 1.0078125]
    assert val[2, 0].tolist() == [4.5, -3.0, -1.25, 0.625]
    assert np.all(val[3] == 0.0)
    assert cu.tolist() == [0, 4 * T]
    assert np.array_equal(kf, vf)


def test_pack_ragged_merge_of_a_frame_with_itself_is_a_copy():
    rng = np.random.default_rng(9)
    k = wl.bf16_bits(rng.standard_normal((1, 12, 2, 8), dtype=np.float32))
    ptr = np.array([0, 2, 3])
    kf_m, _, _ = oc.pack_ragged(k, k, ptr, np.array([[1, 1], [2, 2], [0, 0]]), 4)
    kf_c, _, _ = oc.pack_ragged(k, k, ptr, np.array([[1, -1], [2, -1], [0, -1]]), 4)
    assert np.array_equal(kf_m, kf_c)


def test_planted_packing_mistakes_are_caught(monkeypatch):
    def truncate(x32):
        return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    monkeypatch.setattr(oc, "_bf16_rne", truncate)
    with pytest.raises(AssertionError):
        test_pack_ragged_merge_values_and_rounding()
    monkeypatch.undo()
    real = oc.pack_ragged

    def swapped_heads(k, v, ptr, src, T):
        kf, vf, cu = real(k, v, ptr, src, T)
        return vf, kf, cu                                   # K and V exchanged
    monkeypatch.setattr(oc, "pack_ragged", swapped_heads)
    with pytest.raises(AssertionError):
        test_pack_ragged_copies_equal_the_gathered_frames()


# ---------------------------------------------------------------------------
# latent KV cache (VideoMLA page, method)
# ---------------------------------------------------------------------------
def _mla_inputs(rng, B=1, Nq=5, N=9, H=2, dn=3, dr=2, dc=4, dv=3):
    q = rng.standard_normal((B, Nq, H, dn + dr))
    c = rng.standard_normal((B, N, dc))
    kr = rng.standard_normal((B, N, dr))
    wk = rng.standard_normal((H, dn, dc))
    wv = rng.standard_normal((H, dv, dc))
    return q, c, kr, wk, wv


def test_mla_matches_bruteforce_loops():
    rng = np.random.default_rng(41)
    q, c, kr, wk, wv = _mla_inputs(rng)
    sc = 0.7
    O, L = oc.mla_chunk_attn(q, c, kr, wk, wv, sc)
    B, Nq, H, _ = q.shape
    N, dn, dv = c.shape[1], wk.shape[1], wv.shape[1]
    for h in range(H):
        for i in range(Nq):
            s = []
            for t in range(N):
                k_nope = [math.fsum(wk[h, a, e] * c[0, t, e] for e in range(c.shape[2])) for a in range(dn)]
                key = k_nope + list(kr[0, t])
                s.append(sc * math.fsum(float(q[0, i, h, a]) * key[a] for a in range(len(key))))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            assert abs(L[0, h, i] - (m + math.log(l))) < 1e-12
            for a in range(dv):
                v = [math.fsum(wv[h, a, e] * c[0, t, e] for e in range(c.shape[2])) for t in range(N)]
                assert abs(O[0, i, h, a] - math.fsum(wi * vi for wi, vi in zip(w, v)) / l) < 1e-12


def test_mla_selector_projections_reduce_to_plain_attention():
    # W^K = [I | 0] and W^V = [0 | I] pick latent columns: keys = [c[:, :dn], k^R],
    # values = c[:, dc-dv:], i.e. ordinary attention over explicit arrays
    rng = np.random.default_rng(42)
    dn, dr, dc, dv = 3, 2, 6, 4
    q, c, kr, _, _ = _mla_inputs(rng, dn=dn, dr=dr, dc=dc, dv=dv)
    wk = np.zeros((2, dn, dc)); wv = np.zeros((2, dv, dc))
    for h in range(2):
        wk[h, :, :dn] = np.eye(dn)
        wv[h, :, dc - dv:] = np.eye(dv)
    O, L = oc.mla_chunk_attn(q, c, kr, wk, wv, 0.5)
    for h in range(2):
        K = np.concatenate([c[0, :, :dn], kr[0]], axis=1)
        Oref, Lref = oc.attention(q[0, :, h], K, c[0, :, dc - dv:], 0.5)
        assert np.allclose(O[0, :, h], Oref, atol=1e-12) and np.allclose(L[0, h], Lref, atol=1e-12)


def test_mla_absorbed_query_form_is_equivalent():
    # scores through the absorbed query (W^K_h)^T q^nope against the latent,
    # and outputs through the up-projection of the latent-weighted mean
    rng = np.random.default_rng(43)
    dn, dr = 3, 2
    q, c, kr, wk, wv = _mla_inputs(rng, dn=dn, dr=dr)
    O, L = oc.mla_chunk_attn(q, c, kr, wk, wv, 0.9)
    for h in range(2):
        qt = q[0, :, h, :dn] @ wk[h]                         # [Nq, dc]
        s = 0.9 * (qt @ c[0].T + q[0, :, h, dn:] @ kr[0].T)
        lse = special.logsumexp(s, axis=1)
        p = np.exp(s - lse[:, None])
        assert np.allclose(L[0, h], lse, atol=1e-12)
        assert np.allclose(O[0, :, h], (p @ c[0]) @ wv[h].T, atol=1e-12)


def test_planted_mla_mistakes_are_caught(monkeypatch):
    real = oc.mla_chunk_attn

    def permuted_values(q, c, kr, wk, wv, sc, **kw):
        # value up-projection rows in the wrong order
        return real(q, c, kr, wk, np.asarray(wv)[:, ::-1, :], sc, **kw)
    monkeypatch.setattr(oc, "mla_chunk_attn", permuted_values)
    with pytest.raises(AssertionError):
        test_mla_absorbed_query_form_is_equivalent()
    monkeypatch.undo()

    def rope_dropped(q, c, kr, wk, wv, sc, **kw):
        return real(q, c, np.zeros_like(kr), wk, wv, sc, **kw)
    monkeypatch.setattr(oc, "mla_chunk_attn", rope_dropped)
    with pytest.raises(AssertionError):
        test_mla_matches_bruteforce_loops()

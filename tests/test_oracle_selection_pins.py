"""Pins of the oracle's chunk-mean query and of the wiring of its block-sparse
selection (CPU only).

Sparse Forcing page, section 2: item 1 keeps the top-C blocks by coarse score
as persistent memory, item 2 scores blocks through one representative token
per block, item 3 attends densely to the persistent blocks and sparsely to
the top-K local-window blocks of each query block.  With the readings used
throughout (persistent blocks scored against the mean of the whole query
chunk, local blocks scored per query block against that block's mean query),
the selection has three inputs that a slip could swap: which query
representative scores which candidate range, and over which axes the means
run.

The planted inputs below give every query block of a head its own direction,
so that the chunk-mean ranking of the history blocks differs from every
per-query-block ranking, every query block's local top-K differs, and the two
heads differ.  Expected ids are written out by hand.  A second pin recomputes
the whole selection from raw tokens with math.fsum and Python's sort on
random inputs.  The planted-mistake tests at the end show that each plausible
wiring slip fails these pins.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import chunk_attention as oc

# Small frame-aligned layout: frames of 10 tokens cut into blocks of 4, 4, 2
# (3 blocks per frame).  KV cache: 6 frames = 18 blocks: sink 0-2 (frame 0),
# history 3-11 (frames 1-3), local window 12-17 (frames 4-5, the chunk).
# Query chunk: 2 frames = 6 query blocks of lengths 4, 4, 2, 4, 4, 2.
FT, BLK, D, H = 10, 4, 8, 2
LAYOUT = {"sink_begin": 0, "sink_count": 3, "hist_begin": 3, "hist_count": 9,
          "local_begin": 12, "local_count": 6, "C": 3, "K": 2}
# direction of query block qb in head h: e_qb in head 0, e_(5 - qb) in head 1
Q_DIR = [[0, 1, 2, 3, 4, 5], [5, 4, 3, 2, 1, 0]]
# history blocks 3..11: each a pure direction times a magnitude
HIST = {3: (2, 10.0), 4: (0, 4.0), 5: (1, 6.0), 6: (5, 9.0), 7: (3, 5.5), 8: (4, 3.0),
        9: (2, 1.0), 10: (0, 7.0), 11: (3, 2.0)}


def _planted():
    """Q [1, 20, 2, 8] and K [1, 60, 2, 8]: every token of a block carries its
    block's planted vector, so block means are the planted vectors exactly."""
    spans_q = oc.block_spans(2 * FT, BLK, FT)
    spans_k = oc.block_spans(6 * FT, BLK, FT)
    Q = np.zeros((1, 2 * FT, H, D), np.float32)
    K = np.zeros((1, 6 * FT, H, D), np.float32)
    for h in range(H):
        for qb, (s, l) in enumerate(spans_q):
            Q[0, s:s + l, h, Q_DIR[h][qb]] = 1.0
        for blk, (dim, a) in HIST.items():
            s, l = spans_k[blk]
            K[0, s:s + l, h, dim] = a
        # local block 12 + i: 5 in dimension i, 3 in dimension i - 1 (mod 6),
        # so the query block of direction j scores local block 12 + j at 5,
        # block 12 + (j + 1) % 6 at 3 and every other at 0
        for i in range(6):
            s, l = spans_k[12 + i]
            K[0, s:s + l, h, i] = 5.0
            K[0, s:s + l, h, (i - 1) % 6] = 3.0
        # sink blocks: a value no selection may see
        K[0, 0:FT, h, :] = 50.0
    return Q, K


# Hand-derived expectations.
# Chunk mean of head 0 = (4 e0 + 4 e1 + 2 e2 + 4 e3 + 4 e4 + 2 e5) / 20, so the
# history scores are 3: 1.0, 4: 0.8, 5: 1.2, 6: 0.9, 7: 1.1, 8: 0.6, 9: 0.1,
# 10: 1.4, 11: 0.4 -> top 3 = {5, 7, 10}.  Head 1's chunk mean weighs the
# dimensions (0.1, 0.2, 0.2, 0.1, 0.2, 0.2): 3: 2.0, 4: 0.4, 5: 1.2, 6: 1.8,
# 7: 0.55, 8: 0.6, 9: 0.2, 10: 0.7, 11: 0.2 -> top 3 = {3, 5, 6}.
EXPECT_PERSISTENT = {0: [5, 7, 10], 1: [3, 5, 6]}


def expect_local(h, qb):
    j = Q_DIR[h][qb]
    return sorted([12 + j, 12 + (j + 1) % 6])


def expect_row(h, qb):
    return sorted(set(range(3)) | set(EXPECT_PERSISTENT[h]) | set(expect_local(h, qb)))


# --------------------------------------------------------------------------
# chunk-mean query
# --------------------------------------------------------------------------
def check_chunk_mean(fn):
    # ramp over tokens plus distinct per-(batch, head, channel) offsets: the
    # mean over the N tokens of n + c is (N - 1) / 2 + c
    B, N, Hh, d = 2, 37, 3, 5
    off = (1000.0 * np.arange(B)[:, None, None] + 100.0 * np.arange(Hh)[None, :, None]
           + 10.0 * np.arange(d)[None, None, :])
    x = np.arange(N, dtype=np.float64)[None, :, None, None] + off[:, None, :, :]
    m = np.asarray(fn(x.astype(np.float32)))
    assert m.shape == (B, Hh, 1, d)
    np.testing.assert_allclose(m[:, :, 0, :], (N - 1) / 2.0 + off, rtol=0, atol=1e-9)
    # token mean, not a mean of frame-aligned block means: the planted query
    # chunk has blocks of 4, 4, 2, 4, 4, 2 tokens
    Q, _ = _planted()
    m = np.asarray(fn(Q))
    np.testing.assert_allclose(m[0, 0, 0, :6], [0.2, 0.2, 0.1, 0.2, 0.2, 0.1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(m[0, 1, 0, :6], [0.1, 0.2, 0.2, 0.1, 0.2, 0.2], rtol=0, atol=1e-12)
    # brute force with math.fsum on random data
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 23, 2, 3)).astype(np.float32)
    m = np.asarray(fn(x))
    for h, c in itertools.product(range(2), range(3)):
        assert m[0, h, 0, c] == pytest.approx(math.fsum(float(t) for t in x[0, :, h, c]) / 23,
                                              abs=1e-15)


def test_chunk_mean_query_pins():
    check_chunk_mean(oc.chunk_mean_query)


# --------------------------------------------------------------------------
# selection wiring
# --------------------------------------------------------------------------
def check_selection_planted(select):
    Q, K = _planted()
    sel = select(Q, K, BLK, FT, BLK, FT, dict(LAYOUT))
    for h in range(H):
        assert sel["persistent"]["idx"][0, h, 0].tolist() == EXPECT_PERSISTENT[h], h
        for qb in range(6):
            assert sel["local"]["idx"][0, h, qb].tolist() == expect_local(h, qb), (h, qb)
            r = h * 6 + qb
            row = sel["indices"][sel["indptr"][r]:sel["indptr"][r + 1]].tolist()
            assert row == expect_row(h, qb), (h, qb, row)


def _fsum_mean(x, s, l):
    return [math.fsum(float(t) for t in x[s:s + l, c]) / l for c in range(x.shape[1])]


def _f32_dot(a, b):
    return float(np.float32(math.fsum(float(np.float32(u)) * float(np.float32(v))
                                      for u, v in zip(a, b))))


def _python_topk(scores, cand, K):
    order = sorted(range(len(cand)), key=lambda j: (-scores[j], cand[j]))
    return sorted(cand[j] for j in order[:K])


def check_selection_bruteforce(select):
    """The whole selection recomputed from raw tokens: fsum block and chunk
    means (rounded to float32, the precision block means are handed over
    in), float32-rounded fsum scores, Python's stable sort."""
    rng = np.random.default_rng(8)
    Hh, d, ft, blk = 3, 6, 7, 3               # blocks of 3, 3, 1 tokens per frame
    nf_kv, nf_q = 7, 2
    Q = rng.standard_normal((1, nf_q * ft, Hh, d)).astype(np.float32)
    K = rng.standard_normal((1, nf_kv * ft, Hh, d)).astype(np.float32)
    bpf = 3
    lay = {"sink_begin": 0, "sink_count": bpf, "hist_begin": bpf, "hist_count": 4 * bpf,
           "local_begin": 5 * bpf, "local_count": 2 * bpf, "C": 5, "K": 2}
    sel = select(Q, K, blk, ft, blk, ft, dict(lay))
    sq = oc.block_spans(nf_q * ft, blk, ft).tolist()
    sk = oc.block_spans(nf_kv * ft, blk, ft).tolist()
    for h in range(Hh):
        qh, kh = Q[0, :, h, :], K[0, :, h, :]
        km = [[float(np.float32(v)) for v in _fsum_mean(kh, s, l)] for s, l in sk]
        cm = [float(np.float32(v)) for v in _fsum_mean(qh, 0, len(qh))]
        hist = list(range(lay["hist_begin"], lay["hist_begin"] + lay["hist_count"]))
        pers = _python_topk([_f32_dot(cm, km[j]) for j in hist], hist, lay["C"])
        assert sel["persistent"]["idx"][0, h, 0].tolist() == pers, h
        loc_ids = list(range(lay["local_begin"], lay["local_begin"] + lay["local_count"]))
        for qb, (s, l) in enumerate(sq):
            qm = [float(np.float32(v)) for v in _fsum_mean(qh, s, l)]
            loc = _python_topk([_f32_dot(qm, km[j]) for j in loc_ids], loc_ids, lay["K"])
            assert sel["local"]["idx"][0, h, qb].tolist() == loc, (h, qb)
            r = h * len(sq) + qb
            row = sel["indices"][sel["indptr"][r]:sel["indptr"][r + 1]].tolist()
            assert row == sorted(set(range(bpf)) | set(pers) | set(loc)), (h, qb)


def test_sparse_selection_planted_wiring():
    check_selection_planted(oc.sparse_selection)


def test_sparse_selection_matches_bruteforce():
    check_selection_bruteforce(oc.sparse_selection)


# --------------------------------------------------------------------------
# planted mistakes: each must fail one of the pins above
# --------------------------------------------------------------------------
def _mean_over_heads(Q):
    m = np.asarray(Q, np.float64).mean(axis=(1, 2))[:, None, None, :]
    return np.broadcast_to(m, (Q.shape[0], Q.shape[2], 1, Q.shape[3]))


def _mean_of_block_means(Q):
    # unweighted average of frame-aligned block means (drops the block lengths)
    bm = oc.block_mean(Q, BLK, FT)
    return bm.mean(axis=2)[:, :, None, :]


def _mean_over_channels(Q):
    m = np.asarray(Q, np.float64).mean(axis=(1, 3))
    return np.repeat(m[:, :, None, None], Q.shape[3], axis=3)


@pytest.mark.parametrize("bad", [_mean_over_heads, _mean_of_block_means, _mean_over_channels])
def test_planted_chunk_mean_mistakes_are_caught(bad):
    with pytest.raises(AssertionError):
        check_chunk_mean(bad)


def _selection(local_q, pers_q, head_mean=False):
    """sparse_selection with its query representatives chosen by the caller:
    local_q / pers_q in {"block", "chunk", "block0"}."""
    def select(Q, K, q_block, q_seg, kv_block, kv_seg, layout):
        if head_mean:
            Q = np.broadcast_to(np.asarray(Q).mean(axis=2, keepdims=True), Q.shape)
        B = Q.shape[0]
        qm = oc.block_mean(Q, q_block, q_seg).astype(np.float32)
        km = oc.block_mean(K, kv_block, kv_seg).astype(np.float32)
        cm = oc.chunk_mean_query(Q).astype(np.float32)
        pick = {"block": qm, "chunk": np.broadcast_to(cm, qm.shape).copy(),
                "block0": qm[:, :, :1, :].copy()}
        pq = {"chunk": cm, "block0": qm[:, :, :1, :].copy(), "block": qm[:, :, :1, :].copy()}
        pers = oc.block_score_topk(pq[pers_q], km, layout["hist_begin"], layout["hist_count"],
                                   layout["C"])
        lq = pick[local_q]
        if local_q == "block0":
            lq = np.broadcast_to(lq, qm.shape).copy()
        loc = oc.block_score_topk(lq, km, layout["local_begin"], layout["local_count"],
                                  layout["K"])
        indptr, indices = oc.build_kv_index(B, Q.shape[2], qm.shape[2], layout["sink_begin"],
                                            layout["sink_count"], pers["idx"][:, :, 0, :],
                                            loc["idx"], 0)
        return {"persistent": pers, "local": loc, "indptr": indptr, "indices": indices}
    return select


def test_selection_harness_reproduces_the_oracle():
    # the mutant factory with the right choices passes the pins, so the
    # failures below come from the planted slips alone
    good = _selection("block", "chunk")
    check_selection_planted(good)
    check_selection_bruteforce(good)


@pytest.mark.parametrize("mutant", [
    _selection("chunk", "chunk"),          # local top-K scored against the chunk mean
    _selection("block", "block0"),         # persistent set scored against query block 0
    _selection("block0", "chunk"),         # every query block takes query block 0's top-K
    _selection("block", "chunk", head_mean=True),   # queries averaged over heads
])
def test_planted_selection_wiring_mistakes_are_caught(mutant):
    caught = 0
    for check in (check_selection_planted, check_selection_bruteforce):
        try:
            check(mutant)
        except AssertionError:
            caught += 1
    assert caught == 2

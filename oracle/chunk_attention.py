"""CPU oracle for chunk attention against a video-generation KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or table generators) and never
imports it; the two meet only in the seeded input generators.

Everything here is the plain, slow definition, written for a reader to check
against the pages by eye:

* attention of a query chunk over an explicit key set I, emitting O and the
  natural-log log-sum-exp (LSE) -- ISPA page (Instance-Specific Parametric
  Absorption), section 2 "dual-stream warmup": attention is split into a local
  and a history branch whose LSE states let the two be recombined afterwards;
* the LSE merge of two such branches -- same passage;
* the key set of each cache mode: dense; block-sparse = persistent blocks
  (dense) plus the top-K blocks of the local window -- Sparse Forcing page,
  section 2 items 1-3 (structured memory decomposition, blockified
  compression, PBSA); ragged per-head caches stored flat with boundary
  indices -- Pyramid Forcing page, section 3 "ragged-cache attention";
* block representatives (one token per block: the mean) and coarse scoring
  by representative dot products, followed by exact top-K -- Sparse Forcing
  page, section 2 item 2 and item 1 "memory management", including the
  persistent-set update when blocks leave the local window;
* per-head frame selections and adjacent-frame merges packed into flat
  buffers with boundary indices -- Pyramid Forcing page, sections 2-3;
* attention over a latent KV cache: every head's keys and values rebuilt
  from the shared content latent and rotated position key by the head's
  up-projections, then plain attention -- VideoMLA page, method.

Floating point: inputs are bf16 values given as exactly equal float32 arrays;
attention, merge and block means are computed in float64.  Where a floating
point value decides an integer (the top-K block ids) the decision is taken on
float32 scores, the precision the GPU kernels compute them in.

Parity status: each function below is pinned by tests that do not re-run its
own formula, and planted-mistake tests show the pins catch plausible slips:
  attention, chunk_attn_dense/_blocks/_varlen  brute-force fsum loops, closed
      forms, scipy logsumexp/softmax, all blocks = dense, ragged = gathered
      frames = block lists (tests/test_oracle_pins.py)
  lse_merge, lse_merge_bshd    merge of disjoint branches = attention over
      their union, special cases (tests/test_oracle_pins.py)
  block_spans, block_mean      frame-aligned tiling by hand, ramp and constant
      closed forms, fsum brute force (tests/test_oracle_pins.py)
  chunk_mean_query             ramp with per-(batch, head, channel) offsets,
      planted block lengths, fsum brute force
      (tests/test_oracle_selection_pins.py)
  block_score_topk, persistent_update   planted orders and ties, Python sort
      on fsum scores (tests/test_oracle_pins.py)
  build_kv_index               the set definition (tests/test_oracle_pins.py)
  sparse_selection             planted inputs with hand-derived ids, and the
      whole selection recomputed from raw tokens (fsum, Python sort)
      (tests/test_oracle_selection_pins.py)
  pack_ragged                  gathered frames, hand-rounded merges
  mla_chunk_attn               brute-force loops, reduction to plain
      attention, the absorbed form (tests/test_oracle_pins.py)
No function is left parity unpinned.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Block tiling (Sparse Forcing page, section 2 item 2: the latent is cut into
# spatio-temporal blocks; here each segment -- a latent frame -- is cut into
# block_size-token blocks, the last block of a segment taking the remainder).
# ---------------------------------------------------------------------------
def block_spans(n_tokens: int, block_size: int, seg_len: int) -> np.ndarray:
    """(start, length) of every block, in block-id order, as int64 [NB, 2]."""
    spans: List[Tuple[int, int]] = []
    seg_start = 0
    while seg_start < n_tokens:
        seg_end = min(seg_start + seg_len, n_tokens)
        s = seg_start
        while s < seg_end:
            spans.append((s, min(block_size, seg_end - s)))
            s += block_size
        seg_start = seg_end
    return np.array(spans, dtype=np.int64).reshape(-1, 2)


def block_tokens(spans: np.ndarray, ids: Sequence[int]) -> np.ndarray:
    """Token positions covered by the listed blocks, in list order."""
    parts = [np.arange(spans[i, 0], spans[i, 0] + spans[i, 1]) for i in ids]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------
# Attention over an explicit key set (ISPA page, section 2 item 1: attention
# with its LSE state; the same exact attention is what the PBSA and varlen
# kernels compute over their key sets).
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float
              ) -> Tuple[np.ndarray, np.ndarray]:
    """O_i = sum_j softmax_j(scale * q_i . k_j) v_j and
    LSE_i = ln sum_j exp(scale * q_i . k_j), for q [n, d], k, v [m, d].

    Evaluated in float64; the row maximum is subtracted before exp only to
    keep exp finite (it cancels exactly in O and is added back to the LSE).
    An empty key set gives O = 0 and LSE = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((n, v.shape[1])), np.full(n, NEG_INF)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def _rows(Nq: int, rows: Optional[Sequence[int]]) -> np.ndarray:
    return np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)


def chunk_attn_dense(Q, K, V, scale: float, rows=None, heads=None):
    """Dense cache: every query row attends to all Nkv cached tokens.
    Q [B, Nq, H, d], K/V [B, Nkv, H, d] -> O [B, R, H', d], LSE [B, H', R]
    for the selected rows R (all by default) and heads H' (all by default)."""
    B, Nq, H, d = Q.shape
    r = _rows(Nq, rows)
    hs = list(range(H)) if heads is None else list(heads)
    O = np.zeros((B, len(r), len(hs), V.shape[-1]))
    L = np.full((B, len(hs), len(r)), NEG_INF)
    for b in range(B):
        for j, h in enumerate(hs):
            O[b, :, j], L[b, j] = attention(Q[b, r, h], K[b, :, h], V[b, :, h], scale)
    return O, L


def chunk_attn_blocks(Q, K, V, indptr, indices, kv_block: int, kv_seg: int,
                      q_block: int, q_seg: int, scale: float, rows=None, heads=None):
    """Block-list cache (PBSA, Sparse Forcing page section 2 item 3): the
    query rows of query block qb of head (b, h) attend to the tokens of the
    blocks listed in CSR row (b*H + h)*NQB + qb.  Block ids refer to the
    KV tiling (kv_block, kv_seg); query blocks to the tiling (q_block, q_seg)."""
    B, Nq, H, d = Q.shape
    kv_spans = block_spans(K.shape[1], kv_block, kv_seg)
    q_spans = block_spans(Nq, q_block, q_seg)
    nqb = len(q_spans)
    r = _rows(Nq, rows)
    hs = list(range(H)) if heads is None else list(heads)
    qb_of_row = np.zeros(Nq, dtype=np.int64)
    for qb, (s, l) in enumerate(q_spans):
        qb_of_row[s:s + l] = qb
    O = np.zeros((B, len(r), len(hs), V.shape[-1]))
    L = np.full((B, len(hs), len(r)), NEG_INF)
    for b in range(B):
        for j, h in enumerate(hs):
            for qb in np.unique(qb_of_row[r]):
                sel = np.nonzero(qb_of_row[r] == qb)[0]
                row = (b * H + h) * nqb + int(qb)
                ids = indices[indptr[row]:indptr[row + 1]]
                tok = block_tokens(kv_spans, ids)
                o, l = attention(Q[b, r[sel], h], K[b, tok, h], V[b, tok, h], scale)
                O[b, sel, j] = o
                L[b, j, sel] = l
    return O, L


def chunk_attn_varlen(Q, K_flat, V_flat, cu_seqlens, scale: float, rows=None, heads=None):
    """Ragged per-head cache (Pyramid Forcing page, section 3): head (b, h)
    owns rows [cu[b*H+h], cu[b*H+h+1]) of the flat K/V buffers; no padding."""
    B, Nq, H, d = Q.shape
    r = _rows(Nq, rows)
    hs = list(range(H)) if heads is None else list(heads)
    O = np.zeros((B, len(r), len(hs), V_flat.shape[-1]))
    L = np.full((B, len(hs), len(r)), NEG_INF)
    for b in range(B):
        for j, h in enumerate(hs):
            lo, hi = int(cu_seqlens[b * H + h]), int(cu_seqlens[b * H + h + 1])
            O[b, :, j], L[b, j] = attention(Q[b, r, h], K_flat[lo:hi], V_flat[lo:hi], scale)
    return O, L


# ---------------------------------------------------------------------------
# Ragged cache packing (Pyramid Forcing page, section 2: per-head cache
# policies keep a per-head set of frames -- stride or periodic samples, or
# adjacent frames merged into one -- and section 3: the variable-length caches
# are stored as flat sequences with boundary indices).
# ---------------------------------------------------------------------------
def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (NaN kept
    as a quiet NaN)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def pack_ragged(k_bits, v_bits, frame_ptr, frame_src, frame_tokens: int):
    """Flatten per-head frame selections of a dense cache.

    k_bits, v_bits  uint16 bf16 bit patterns [B, N, H, d] (the dense cache)
    frame_ptr       int [B*H + 1]: head bh owns output frames
                    [frame_ptr[bh], frame_ptr[bh+1]), heads in order
    frame_src       int [F, 2]: output frame j copies source frame a =
                    frame_src[j, 0] of its head, or, when b = frame_src[j, 1]
                    is not -1, merges frames a and b: each element is the
                    float32 sum of the two bf16 values times 1/2, rounded to
                    bf16 (nearest, ties to even).  A source frame outside the
                    cache contributes zeros.
    Returns (k_flat, v_flat) uint16 [F * frame_tokens, d] and cu_seqlens
    int32 [B*H + 1] = frame_ptr * frame_tokens."""
    B, N, H, d = k_bits.shape
    nf = N // frame_tokens
    frame_ptr = np.asarray(frame_ptr, dtype=np.int64)
    frame_src = np.asarray(frame_src, dtype=np.int64).reshape(-1, 2)
    F = int(frame_ptr[-1])
    outs = []
    for src in (k_bits, v_bits):
        flat = np.zeros((F * frame_tokens, d), dtype=np.uint16)
        for bh in range(B * H):
            b, h = divmod(bh, H)
            for j in range(int(frame_ptr[bh]), int(frame_ptr[bh + 1])):
                def frame(f):
                    if 0 <= f < nf:
                        rows = src[b, f * frame_tokens:(f + 1) * frame_tokens, h, :]
                        return (rows.astype(np.uint32) << 16).view(np.float32)
                    return np.zeros((frame_tokens, d), dtype=np.float32)
                a, c = int(frame_src[j, 0]), int(frame_src[j, 1])
                if c == -1:
                    bits = _bf16_rne(frame(a))
                else:
                    s32 = (frame(a) + frame(c)).astype(np.float32)   # one float32 rounding
                    bits = _bf16_rne((s32 * np.float32(0.5)).astype(np.float32))
                flat[j * frame_tokens:(j + 1) * frame_tokens] = bits
        outs.append(flat)
    cu = (frame_ptr * frame_tokens).astype(np.int32)
    return outs[0], outs[1], cu


# ---------------------------------------------------------------------------
# Latent KV cache (VideoMLA page, method): the cache keeps per token a content
# latent c_t (d_c values shared by all heads) and one rotated position key
# k^R_t (d_rope values, shared by all heads).  Head h reconstructs its keys
# and values on demand with up-projections: k_{t,h} = [W^K_h c_t ; k^R_t]
# (content part d_nope = W^K_h's rows, position part d_rope) and
# v_{t,h} = W^V_h c_t.  Queries carry the same split [q^nope ; q^R].
# ---------------------------------------------------------------------------
def mla_chunk_attn(q, c_kv, k_rope, w_uk, w_uv, scale: float, rows=None, heads=None):
    """q [B, Nq, H, d_nope + d_rope], c_kv [B, N, d_c], k_rope [B, N, d_rope],
    w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c] -> O [B, R, H', d_v], LSE
    [B, H', R]: for each head the keys and values are reconstructed from the
    latent cache and attended with plain softmax attention."""
    q = np.asarray(q, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Nq, H, _ = q.shape
    r = _rows(Nq, rows)
    hs = list(range(H)) if heads is None else list(heads)
    d_v = w_uv.shape[1]
    O = np.zeros((B, len(r), len(hs), d_v))
    L = np.full((B, len(hs), len(r)), NEG_INF)
    for b in range(B):
        for j, h in enumerate(hs):
            k_h = np.concatenate([c_kv[b] @ w_uk[h].T, k_rope[b]], axis=1)   # [N, d_nope + d_rope]
            v_h = c_kv[b] @ w_uv[h].T                                         # [N, d_v]
            O[b, :, j], L[b, j] = attention(q[b, r, h], k_h, v_h, scale)
    return O, L


# ---------------------------------------------------------------------------
# LSE merge (ISPA page, section 2 item 1: local and history branches combined
# after the fact through their LSE states).
# ---------------------------------------------------------------------------
def lse_merge(o1, lse1, o2, lse2) -> Tuple[np.ndarray, np.ndarray]:
    """Combine two attention results over disjoint key sets.
    o* [..., d], lse* [...] (o's leading shape).  With M = max(lse1, lse2)
    and w_k = exp(lse_k - M): LSE = M + ln(w1 + w2),
    O = (w1 O1 + w2 O2) / (w1 + w2).  Both branches empty -> O = 0, -inf."""
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    l1 = np.asarray(lse1, dtype=np.float64)
    l2 = np.asarray(lse2, dtype=np.float64)
    M = np.maximum(l1, l2)
    live = M > NEG_INF
    Ms = np.where(live, M, 0.0)
    w1 = np.where(live, np.exp(l1 - Ms), 0.0)
    w2 = np.where(live, np.exp(l2 - Ms), 0.0)
    tot = w1 + w2
    lse = np.where(live, Ms + np.log(np.where(live, tot, 1.0)), NEG_INF)
    den = np.where(live, tot, 1.0)[..., None]
    o = (w1[..., None] * o1 + w2[..., None] * o2) / den
    return np.where(live[..., None], o, 0.0), lse


def lse_merge_bshd(O1, L1, O2, L2):
    """lse_merge for O in [B, N, H, d] and LSE in [B, H, N] layout."""
    o, l = lse_merge(O1, np.transpose(L1, (0, 2, 1)), O2, np.transpose(L2, (0, 2, 1)))
    return o, np.transpose(l, (0, 2, 1))


# ---------------------------------------------------------------------------
# Block representatives and coarse scoring (Sparse Forcing page, section 2
# item 2 "blockified compression": each block becomes one representative
# token used for coarse-grained scoring; the representative is the mean).
# ---------------------------------------------------------------------------
def block_mean(x, block_size: int, seg_len: int) -> np.ndarray:
    """x [B, N, H, d] -> [B, H, NB, d] float64: mean of each block's tokens."""
    B, N, H, d = x.shape
    spans = block_spans(N, block_size, seg_len)
    out = np.zeros((B, H, len(spans), d))
    x64 = np.asarray(x, dtype=np.float64)
    for j, (s, l) in enumerate(spans):
        out[:, :, j, :] = x64[:, s:s + l].sum(axis=1) / l
    return out


def chunk_mean_query(Q) -> np.ndarray:
    """Mean of all chunk queries per head: [B, Nq, H, d] -> [B, H, 1, d]."""
    return np.asarray(Q, dtype=np.float64).mean(axis=1)[:, :, None, :]


def block_score_topk(q_mean, k_mean, cand_begin: int, cand_count: int, K: int,
                     tie_eps: float = 1e-4) -> Dict[str, np.ndarray]:
    """Coarse scores sigma(qb, c) = <q_mean[qb], k_mean[c]> over the candidate
    blocks c in [cand_begin, cand_begin + cand_count), then the K best per
    (b, h, qb): higher score first, equal scores -> lower block id first.
    The chosen ids are returned ascending.

    Block means arrive as the float32 values the kernels produce; each score
    is the float64 dot product rounded once to float32, and the ordering
    decision is taken on those float32 values.

    Returns idx [B, H, NQB, K] int32, score [B, H, NQB, K] float32 (in idx
    order), gap [B, H, NQB] = score of K-th best minus (K+1)-th best (inf if
    K == cand_count), near_tie [B, H, NQB] = number of candidates whose
    score is within tie_eps of the K-th best (the K-th itself included),
    kth [B, H, NQB] = the K-th best score, and every candidate's id and
    score: cand [B, H, NQB, cand_count] int64, cand_score (same shape,
    float32), so that a selection differing at near-ties can be checked."""
    qm = np.asarray(q_mean, dtype=np.float32).astype(np.float64)
    km = np.asarray(k_mean, dtype=np.float32).astype(np.float64)
    B, H, NQB, d = qm.shape
    if not 1 <= K <= cand_count:
        raise ValueError("need 1 <= K <= cand_count")
    cand = np.arange(cand_begin, cand_begin + cand_count)
    idx = np.zeros((B, H, NQB, K), dtype=np.int32)
    sc = np.zeros((B, H, NQB, K), dtype=np.float32)
    gap = np.full((B, H, NQB), np.inf)
    near = np.zeros((B, H, NQB), dtype=np.int64)
    kth_all = np.zeros((B, H, NQB))
    cand_score = np.zeros((B, H, NQB, cand_count), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            kc = km[b, h, cand]
            for qb in range(NQB):
                s = (kc @ qm[b, h, qb]).astype(np.float32)
                cand_score[b, h, qb] = s
                order = np.lexsort((cand, -s.astype(np.float64)))
                top = order[:K]
                asc = top[np.argsort(cand[top])]
                idx[b, h, qb] = cand[asc]
                sc[b, h, qb] = s[asc]
                kth = float(s[order[K - 1]])
                kth_all[b, h, qb] = kth
                if K < cand_count:
                    gap[b, h, qb] = kth - float(s[order[K]])
                near[b, h, qb] = int(np.sum(np.abs(s.astype(np.float64) - kth) < tie_eps))
    return {"idx": idx, "score": sc, "gap": gap, "near_tie": near, "kth": kth_all,
            "cand": np.broadcast_to(cand, (B, H, NQB, cand_count)).copy(),
            "cand_score": cand_score}


def persistent_update(q_mean, k_mean, persistent, evict_begin: int, evict_count: int, C: int,
                      tie_eps: float = 1e-4) -> Dict[str, np.ndarray]:
    """Persistent-memory update when the local window slides (Sparse Forcing
    page, section 2 item 1, memory management): the blocks evicted from the
    local window, [evict_begin, evict_begin + evict_count), join the head's
    current persistent blocks as candidates, and the C best by coarse score
    against the query representative q_mean [B, H, 1, d] (the chunk-mean
    query) form the new persistent set.

    Candidates are the set union: a persistent id inside the evicted range,
    or outside [0, NB), is not a second candidate.  Scores, ordering and tie
    rule as in block_score_topk (float32 scores, higher first, lower id first
    on equal scores); the kept ids are returned ascending, padded with -1 (and
    score -inf) when fewer than C candidates exist.  Also returns gap,
    near_tie and kth as block_score_topk does, and the candidates with their
    scores (cand [B, H, n_max] int64 padded with -1, cand_score padded with
    -inf)."""
    qm = np.asarray(q_mean, dtype=np.float32).astype(np.float64)
    km = np.asarray(k_mean, dtype=np.float32).astype(np.float64)
    pers = np.asarray(persistent, dtype=np.int64)
    B, H, _, d = qm.shape
    NB = km.shape[2]
    ev = set(range(evict_begin, evict_begin + evict_count))
    idx = np.full((B, H, C), -1, dtype=np.int32)
    sc = np.full((B, H, C), -np.inf, dtype=np.float32)
    gap = np.full((B, H), np.inf)
    near = np.zeros((B, H), dtype=np.int64)
    kth_all = np.full((B, H), -np.inf)
    cands = []
    for b in range(B):
        for h in range(H):
            cand = sorted(ev | {int(x) for x in pers[b, h] if 0 <= x < NB})
            cand = np.array(cand, dtype=np.int64)
            s = np.array([np.float32(np.dot(qm[b, h, 0], km[b, h, c])) for c in cand],
                         dtype=np.float32)
            cands.append((cand, s))
            order = np.lexsort((cand, -s.astype(np.float64)))
            k = min(C, len(cand))
            top = order[:k]
            asc = top[np.argsort(cand[top])]
            idx[b, h, :k] = cand[asc]
            sc[b, h, :k] = s[asc]
            if k:
                kth = float(s[order[k - 1]])
                kth_all[b, h] = kth
                if k < len(cand):
                    gap[b, h] = kth - float(s[order[k]])
                near[b, h] = int(np.sum(np.abs(s.astype(np.float64) - kth) < tie_eps))
    n_max = max([len(c) for c, _ in cands] + [0])
    cand_ids = np.full((B, H, n_max), -1, dtype=np.int64)
    cand_sc = np.full((B, H, n_max), -np.inf, dtype=np.float32)
    for i, (c, s) in enumerate(cands):
        cand_ids[i // H, i % H, :len(c)] = c
        cand_sc[i // H, i % H, :len(c)] = s
    return {"idx": idx, "score": sc, "gap": gap, "near_tie": near, "kth": kth_all,
            "cand": cand_ids, "cand_score": cand_sc}


def build_kv_index(B: int, H: int, NQB: int, sink_begin: int, sink_count: int,
                   persistent: Optional[np.ndarray], topk: Optional[np.ndarray],
                   topk_offset: int) -> Tuple[np.ndarray, np.ndarray]:
    """CSR block lists for PBSA (Sparse Forcing page, section 2 item 3: dense
    attention over the persistent blocks, sparse attention over the top-K
    local-window blocks; sink blocks are attended by every query block).
    Row (b*H + h)*NQB + qb = sorted unique union of
    {sink_begin .. sink_begin+sink_count-1}, persistent[b, h, :] and
    {topk_offset + t : t in topk[b, h, qb, :]}."""
    rows: List[np.ndarray] = []
    for b in range(B):
        for h in range(H):
            for qb in range(NQB):
                s = set(range(sink_begin, sink_begin + sink_count))
                if persistent is not None:
                    s |= set(int(x) for x in persistent[b, h])
                if topk is not None:
                    s |= set(int(t) + topk_offset for t in topk[b, h, qb])
                rows.append(np.array(sorted(s), dtype=np.int32))
    indptr = np.zeros(len(rows) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(r) for r in rows])
    indices = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int32)
    return indptr, indices.astype(np.int32)


def sparse_selection(Q, K, q_block: int, q_seg: int, kv_block: int, kv_seg: int,
                     layout: Dict) -> Dict[str, np.ndarray]:
    """The block-sparse selection steps in the Sparse Forcing page's order:
    blockified compression (block means of Q and K), persistent memory = the
    top-C history blocks by coarse score against the chunk-mean query
    (section 2 item 1), top-K local-window blocks per query block by coarse
    score (item 2), then the PBSA block lists (item 3)."""
    B, Nq, H, d = Q.shape
    qm = block_mean(Q, q_block, q_seg).astype(np.float32)
    km = block_mean(K, kv_block, kv_seg).astype(np.float32)
    cm = chunk_mean_query(Q).astype(np.float32)
    pers = block_score_topk(cm, km, layout["hist_begin"], layout["hist_count"], layout["C"])
    loc = block_score_topk(qm, km, layout["local_begin"], layout["local_count"], layout["K"])
    indptr, indices = build_kv_index(B, H, qm.shape[2], layout["sink_begin"],
                                     layout["sink_count"], pers["idx"][:, :, 0, :],
                                     loc["idx"], 0)
    return {"q_mean": qm, "k_mean": km, "chunk_mean": cm, "persistent": pers,
            "local": loc, "indptr": indptr, "indices": indices}

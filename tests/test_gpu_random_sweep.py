"""GPU parity over seeded random configurations of every attention mode, the
LSE merge and block means, against the CPU oracle on the whole output (O
max-abs 1e-2 plus the bf16 output half-ulp from |O| = 2, LSE max-abs 1e-3).

Each case draws its shape, tiling and lists from its own seed: batch and
head counts, d = 64 or 128, query and key lengths from 1 (0 for keys) up to a
few hundred / a thousand and more tokens, frame-aligned tilings with tail
blocks of any length (block sizes 1..64 on the key axis, up to 300 on the
query axis), random CSR lists (empty rows, unsorted ids), disjoint shared /
local lists for one-pass PBSA, ragged per-head lengths including empty heads,
per-head mixed modes, strided head-subset views, bf16 or float32 outputs and
every schedule policy.  Outputs start as NaN, so every element must be
written.  The draw of each case is printed before it runs.
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

N_CASES = 12        # per mode


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _bf(rng, shape, scale):
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def _tensors(rng, B, Nq, Nkv, H, d):
    sq, sk = rng.uniform(0.5, 1.5, size=2)
    return _bf(rng, (B, Nq, H, d), sq), _bf(rng, (B, Nkv, H, d), sk), _bf(rng, (B, Nkv, H, d), 1.0)


def _views(rng, Q, K, V):
    """Device tensors, as head-subset views of wider buffers (every other
    head of 2H + 1) half of the time."""
    H = Q.shape[2]
    if rng.random() < 0.5:
        return to_dev(Q), to_dev(K), to_dev(V)
    def wide(X):
        B, N, _, d = X.shape
        Xw = wl.Bf16Tensor(np.zeros((B, N, 2 * H + 1, d), np.uint16))
        Xw.bits[:, :, 1::2] = X.bits
        return to_dev(Xw)[:, :, 1::2]
    return wide(Q), wide(K), wide(V)


def _csr(rows):
    ip = np.zeros(len(rows) + 1, np.int32)
    ip[1:] = np.cumsum([len(r) for r in rows])
    ix = np.concatenate(rows).astype(np.int32) if ip[-1] else np.zeros(1, np.int32)
    return ip, ix


def _tiling(rng, n, bmax):
    block = int(rng.integers(1, bmax + 1))
    seg = int(rng.integers(block, max(block + 1, 3 * block + 18)))
    return block, max(1, min(seg, max(n, 1)) if rng.random() < 0.2 else seg)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_dense(case):
    rng = np.random.default_rng(7000 + case)
    B, H, d = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    Nq, Nkv = int(rng.integers(1, 400)), int(rng.integers(0, 1600))
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    policy = str(rng.choice(["never", "always", "auto"]))
    say(f"random dense #{case}: B={B} H={H} d={d} Nq={Nq} Nkv={Nkv} out={odt} schedule={policy}")
    Q, K, V = _tensors(rng, B, Nq, Nkv, H, d)
    q, k, v = _views(rng, Q, K, V)
    o, l = nan_out(B, Nq, H, d, odt), nan_lse(B, H, Nq)
    ca.chunk_attn_fwd(q, k, v, out=o, lse=l, balanced=policy)
    torch.cuda.synchronize()
    assert_written("random dense", o, l)
    Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, 1 / math.sqrt(d))
    assert_o(o, Or, odt == torch.bfloat16, f"random dense #{case}")
    assert_lse(l, Lr, f"random dense #{case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_block_lists(case):
    rng = np.random.default_rng(7100 + case)
    B, H, d = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    Nq, Nkv = int(rng.integers(1, 400)), int(rng.integers(1, 1600))
    kvb, kvs = _tiling(rng, Nkv, 64)
    qb, qs = _tiling(rng, Nq, 300)
    nkb, nqb = len(orc.block_spans(Nkv, kvb, kvs)), len(orc.block_spans(Nq, qb, qs))
    rows = [rng.permutation(nkb)[:int(rng.integers(0, min(nkb, 40) + 1))] for _ in range(B * H * nqb)]
    ip, ix = _csr(rows)
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    say(f"random block lists #{case}: B={B} H={H} d={d} Nq={Nq} Nkv={Nkv} kv tiling ({kvb},{kvs}) "
        f"q tiling ({qb},{qs}) rows={len(rows)} nnz={int(ip[-1])} out={odt}")
    Q, K, V = _tensors(rng, B, Nq, Nkv, H, d)
    q, k, v = _views(rng, Q, K, V)
    o, l = nan_out(B, Nq, H, d, odt), nan_lse(B, H, Nq)
    ca.chunk_attn_fwd(q, k, v, kv_indptr=i32(ip), kv_indices=i32(ix), kv_block=kvb, kv_seg=kvs,
                      q_block=qb, q_seg=qs, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("random block lists", o, l)
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, ip, ix, kvb, kvs, qb, qs, 1 / math.sqrt(d))
    assert_o(o, Or, odt == torch.bfloat16, f"random block lists #{case}")
    assert_lse(l, Lr, f"random block lists #{case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_pbsa(case):
    rng = np.random.default_rng(7200 + case)
    B, H, d = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    Nq, Nkv = int(rng.integers(1, 400)), int(rng.integers(1, 1600))
    kvb, kvs = _tiling(rng, Nkv, 64)
    qb, qs = _tiling(rng, Nq, 64)
    nkb, nqb = len(orc.block_spans(Nkv, kvb, kvs)), len(orc.block_spans(Nq, qb, qs))
    shared, local, union = [], [], []
    for _ in range(B * H):
        perm = rng.permutation(nkb)
        ns = int(rng.integers(0, min(nkb, 30) + 1))
        shared.append(perm[:ns])
        rest = perm[ns:]
        for _ in range(nqb):
            loc = rng.permutation(rest)[:int(rng.integers(0, min(len(rest), 12) + 1))]
            local.append(loc)
            union.append(np.concatenate([perm[:ns], loc]))
    sp, sx = _csr(shared)
    lp, lx = _csr(local)
    up, ux = _csr(union)
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    say(f"random PBSA #{case}: B={B} H={H} d={d} Nq={Nq} Nkv={Nkv} kv tiling ({kvb},{kvs}) "
        f"q tiling ({qb},{qs}) shared nnz={int(sp[-1])} local nnz={int(lp[-1])} out={odt}")
    Q, K, V = _tensors(rng, B, Nq, Nkv, H, d)
    q, k, v = _views(rng, Q, K, V)
    o, l = nan_out(B, Nq, H, d, odt), nan_lse(B, H, Nq)
    ca.chunk_attn_pbsa_fwd(q, k, v, i32(sp), i32(sx), i32(lp), i32(lx), kv_block=kvb, kv_seg=kvs,
                           q_block=qb, q_seg=qs, out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("random PBSA", o, l)
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, up, ux, kvb, kvs, qb, qs, 1 / math.sqrt(d))
    assert_o(o, Or, odt == torch.bfloat16, f"random PBSA #{case}")
    assert_lse(l, Lr, f"random PBSA #{case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_ragged(case):
    rng = np.random.default_rng(7300 + case)
    B, H, d = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    Nq = int(rng.integers(1, 400))
    lens = rng.integers(0, 1200, size=B * H)
    lens[rng.random(B * H) < 0.2] = 0
    cu = np.zeros(B * H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    host = bool(rng.random() < 0.6)
    policy = str(rng.choice(["never", "always", "auto"]))
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    say(f"random ragged #{case}: B={B} H={H} d={d} Nq={Nq} lengths={lens.tolist()} host cu={host} "
        f"schedule={policy} out={odt}")
    sq, sk = rng.uniform(0.5, 1.5, size=2)
    Q = _bf(rng, (B, Nq, H, d), sq)
    Kf, Vf = _bf(rng, (max(total, 1), d), sk), _bf(rng, (max(total, 1), d), 1.0)
    Kf, Vf = wl.Bf16Tensor(Kf.bits[:total]), wl.Bf16Tensor(Vf.bits[:total])
    o, l = nan_out(B, Nq, H, d, odt), nan_lse(B, H, Nq)
    ca.chunk_attn_varlen_fwd(to_dev(Q), to_dev(Kf), to_dev(Vf), i32(cu),
                             cu_seqlens_host=cu if host else None, out=o, lse=l, balanced=policy)
    torch.cuda.synchronize()
    assert_written("random ragged", o, l)
    Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, 1 / math.sqrt(d))
    assert_o(o, Or, odt == torch.bfloat16, f"random ragged #{case}")
    assert_lse(l, Lr, f"random ragged #{case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_mixed(case):
    rng = np.random.default_rng(7400 + case)
    B, H, d = 1, int(rng.integers(2, 7)), int(rng.choice([64, 128]))
    Nq, Nkv = int(rng.integers(1, 300)), int(rng.integers(1, 1200))
    mode = rng.integers(0, 3, size=B * H).astype(np.int32)
    kvb, kvs = _tiling(rng, Nkv, 64)
    qb, qs = _tiling(rng, Nq, 128)
    nkb, nqb = len(orc.block_spans(Nkv, kvb, kvs)), len(orc.block_spans(Nq, qb, qs))
    rows = [rng.permutation(nkb)[:int(rng.integers(0, min(nkb, 30) + 1))] for _ in range(B * H * nqb)]
    ip, ix = _csr(rows)
    lens = rng.integers(0, 900, size=B * H)
    cu = np.zeros(B * H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    policy = str(rng.choice(["never", "always", "auto"]))
    say(f"random mixed #{case}: H={H} d={d} Nq={Nq} Nkv={Nkv} modes={mode.tolist()} kv tiling "
        f"({kvb},{kvs}) q tiling ({qb},{qs}) ragged lengths={lens.tolist()} schedule={policy}")
    Q, K, V = _tensors(rng, B, Nq, Nkv, H, d)
    Kf, Vf = _bf(rng, (max(total, 1), d), 1.0), _bf(rng, (max(total, 1), d), 1.0)
    Kf, Vf = wl.Bf16Tensor(Kf.bits[:total]), wl.Bf16Tensor(Vf.bits[:total])
    o, l = nan_out(B, Nq, H, d, torch.bfloat16), nan_lse(B, H, Nq)
    ca.chunk_attn_mixed_fwd(to_dev(Q), mode, k=to_dev(K), v=to_dev(V), kv_indptr=i32(ip),
                            kv_indices=i32(ix), kv_block=kvb, kv_seg=kvs, q_block=qb, q_seg=qs,
                            k_flat=to_dev(Kf), v_flat=to_dev(Vf), cu_seqlens=i32(cu),
                            cu_seqlens_host=cu, out=o, lse=l, balanced=policy)
    torch.cuda.synchronize()
    assert_written("random mixed", o, l)
    og, lg = o.float().cpu().numpy(), l.cpu().numpy()
    sc = 1 / math.sqrt(d)
    for h in range(H):
        if mode[h] == 0:
            Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc, heads=[h])
        elif mode[h] == 1:
            Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, ip, ix, kvb, kvs, qb, qs, sc, heads=[h])
        else:
            Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, sc, heads=[h])
        assert_o(og[:, :, h:h + 1], Or, True, f"random mixed #{case} head {h}")
        assert_lse(lg[:, h:h + 1], Lr, f"random mixed #{case} head {h}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_mixed_pbsa(case):
    """Mixed modes with the block-list heads as one-pass PBSA (shared row per
    head + local row per query block, disjoint)."""
    rng = np.random.default_rng(7600 + case)
    B, H, d = 1, int(rng.integers(2, 7)), int(rng.choice([64, 128]))
    Nq, Nkv = int(rng.integers(1, 300)), int(rng.integers(1, 1200))
    mode = rng.integers(0, 3, size=B * H).astype(np.int32)
    kvb, kvs = _tiling(rng, Nkv, 64)
    qb, qs = _tiling(rng, Nq, 64)
    nkb, nqb = len(orc.block_spans(Nkv, kvb, kvs)), len(orc.block_spans(Nq, qb, qs))
    shared, local, union = [], [], []
    for _ in range(B * H):
        perm = rng.permutation(nkb)
        ns = int(rng.integers(0, min(nkb, 20) + 1))
        shared.append(perm[:ns])
        for _ in range(nqb):
            loc = rng.permutation(perm[ns:])[:int(rng.integers(0, min(nkb - ns, 10) + 1))]
            local.append(loc)
            union.append(np.concatenate([perm[:ns], loc]))
    sp, sx = _csr(shared)
    lp, lx = _csr(local)
    up, ux = _csr(union)
    lens = rng.integers(0, 900, size=B * H)
    cu = np.zeros(B * H + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    policy = str(rng.choice(["never", "always", "auto"]))
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    say(f"random mixed PBSA #{case}: H={H} d={d} Nq={Nq} Nkv={Nkv} modes={mode.tolist()} kv tiling "
        f"({kvb},{kvs}) q tiling ({qb},{qs}) shared nnz={int(sp[-1])} local nnz={int(lp[-1])} "
        f"schedule={policy} out={odt}")
    Q, K, V = _tensors(rng, B, Nq, Nkv, H, d)
    Kf, Vf = _bf(rng, (max(total, 1), d), 1.0), _bf(rng, (max(total, 1), d), 1.0)
    Kf, Vf = wl.Bf16Tensor(Kf.bits[:total]), wl.Bf16Tensor(Vf.bits[:total])
    q, k, v = _views(rng, Q, K, V)
    o, l = nan_out(B, Nq, H, d, odt), nan_lse(B, H, Nq)
    ca.chunk_attn_mixed_fwd(q, mode, k=k, v=v, kv_indptr=i32(lp), kv_indices=i32(lx),
                            kv_shared_indptr=i32(sp), kv_shared_indices=i32(sx), kv_block=kvb,
                            kv_seg=kvs, q_block=qb, q_seg=qs, k_flat=to_dev(Kf), v_flat=to_dev(Vf),
                            cu_seqlens=i32(cu), cu_seqlens_host=cu, out=o, lse=l, balanced=policy)
    torch.cuda.synchronize()
    assert_written("random mixed PBSA", o, l)
    og, lg = o.float().cpu().numpy(), l.cpu().numpy()
    sc = 1 / math.sqrt(d)
    for h in range(H):
        if mode[h] == 0:
            Or, Lr = orc.chunk_attn_dense(Q.f32, K.f32, V.f32, sc, heads=[h])
        elif mode[h] == 1:
            Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, up, ux, kvb, kvs, qb, qs, sc, heads=[h])
        else:
            Or, Lr = orc.chunk_attn_varlen(Q.f32, Kf.f32, Vf.f32, cu, sc, heads=[h])
        assert_o(og[:, :, h:h + 1], Or, odt == torch.bfloat16, f"random mixed PBSA #{case} head {h}")
        assert_lse(lg[:, h:h + 1], Lr, f"random mixed PBSA #{case} head {h}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_merge_and_block_means(case):
    rng = np.random.default_rng(7500 + case)
    B, H, d = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    N = int(rng.integers(1, 500))
    idt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    odt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    block, seg = _tiling(rng, N, 64)
    say(f"random merge / block means #{case}: B={B} H={H} d={d} N={N} in={idt} out={odt} "
        f"tiling ({block},{seg})")
    O1 = rng.standard_normal((B, N, H, d)).astype(np.float32)
    O2 = rng.standard_normal((B, N, H, d)).astype(np.float32)
    L1 = (rng.standard_normal((B, H, N)) * 4).astype(np.float32)
    L2 = (rng.standard_normal((B, H, N)) * 4).astype(np.float32)
    L1[rng.random((B, H, N)) < 0.1] = -np.inf
    L2[rng.random((B, H, N)) < 0.1] = -np.inf
    o1 = torch.from_numpy(O1).cuda().to(idt)
    o2 = torch.from_numpy(O2).cuda().to(idt)
    l1, l2 = torch.from_numpy(L1).cuda(), torch.from_numpy(L2).cuda()
    out, lo = nan_out(B, N, H, d, odt), nan_lse(B, H, N)
    ca.lse_merge(o1, l1, o2, l2, out=out, out_lse=lo)
    torch.cuda.synchronize()
    assert_written("random merge", out, lo)
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    Om, Lm = orc.lse_merge_bshd(f64(o1), L1, f64(o2), L2)
    assert_o(out, Om, odt == torch.bfloat16, f"random merge #{case}")
    assert_lse(lo, Lm, f"random merge #{case}")
    X = _bf(rng, (B, N, H, d), 2.0)
    m = ca.block_mean(to_dev(X), block, seg)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().numpy(), orc.block_mean(X.f32, block, seg), rtol=0, atol=2e-6)

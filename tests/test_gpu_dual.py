"""GPU parity of the dual-output pass (ISPA page, section 2 item 1: local
branch = sink + current frames, full branch = the whole cache, computed side
by side): one block-list pass writes attention over each row's first
local_count blocks and over the whole row.  Both are checked against the CPU
oracle's attention over the corresponding block lists."""
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


def _prefix_csr(indptr, indices, n):
    """CSR of the first n ids of every row."""
    rows = [indices[indptr[r]:indptr[r + 1]][:n] for r in range(len(indptr) - 1)]
    ip = np.zeros(len(rows) + 1, np.int32)
    ip[1:] = np.cumsum([len(x) for x in rows])
    ix = np.concatenate(rows).astype(np.int32) if ip[-1] else np.zeros(0, np.int32)
    return ip, ix


@pytest.mark.parametrize("d,local_count,out_dtype", [
    (128, 3, torch.bfloat16), (64, 0, torch.float32), (128, 7, torch.float32), (64, 100, torch.bfloat16),
])
def test_dual_random_lists(d, local_count, out_dtype):
    say(f"dual random lists d={d} local={local_count}")
    B, H, Nq, Nkv, seg, blk = 2, 2, 200, 500, 100, 64
    Q, K, V = _gen(1, (B, Nq, H, d), 1.5), _gen(2, (B, Nkv, H, d), 1.5), _gen(3, (B, Nkv, H, d))
    nkb = orc.block_spans(Nkv, blk, seg).shape[0]
    nqb = orc.block_spans(Nq, blk, seg).shape[0]
    rng = np.random.default_rng(d + local_count)
    lists = [rng.permutation(nkb)[:rng.integers(0, nkb + 1)] for _ in range(B * H * nqb)]
    ip = np.zeros(len(lists) + 1, np.int32)
    ip[1:] = np.cumsum([len(x) for x in lists])
    ix = np.concatenate(lists).astype(np.int32)
    ol, ll, o, l = ca.chunk_attn_dual_fwd(to_dev(Q), to_dev(K), to_dev(V), i32(ip), i32(ix),
                                          local_count, kv_block=blk, kv_seg=seg, q_block=blk,
                                          q_seg=seg, out_dtype=out_dtype)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(d)
    lp, lx = _prefix_csr(ip, ix, local_count)
    Orl, Lrl = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, lp, lx, blk, seg, blk, seg, sc)
    Or, Lr = orc.chunk_attn_blocks(Q.f32, K.f32, V.f32, ip, ix, blk, seg, blk, seg, sc)
    bf = out_dtype == torch.bfloat16
    assert_o(ol, Orl, bf, "dual local")
    assert_lse(ll, Lrl, "dual local")
    assert_o(o, Or, bf, "dual full")
    assert_lse(l, Lr, "dual full")


def test_dual_wan_local_and_full(wan=None):
    say("dual wan: local (sink + chunk frames) and full cache in one pass")
    w = wl.wan_dense(seed=0)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    local, hist = w.meta["local_blocks"], w.meta["history_blocks"]
    row = np.array(local + hist, np.int32)
    ip = np.arange(w.H + 1, dtype=np.int32) * len(row)
    ix = np.tile(row, w.H)
    ol, o = (nan_out(1, w.Nq, w.H, w.d, torch.float32) for _ in range(2))
    ll, l = nan_lse(1, w.H, w.Nq), nan_lse(1, w.H, w.Nq)
    ca.chunk_attn_dual_fwd(q, k, v, i32(ip), i32(ix), len(local), kv_block=64, kv_seg=1560,
                           q_block=w.Nq, q_seg=w.Nq, scale=w.scale, out_local=ol, lse_local=ll,
                           out=o, lse=l)
    torch.cuda.synchronize()
    assert_written("wan dual", ol, ll, o, l)
    rows = wave_rows(w.Nq, seed=5)
    tok = orc.block_tokens(orc.block_spans(w.Nkv, 64, 1560), local)
    Orl, Lrl = orc.chunk_attn_dense(w.q.f32[:, rows], w.k.f32[:, tok], w.v.f32[:, tok], w.scale)
    Or, Lr = orc.chunk_attn_dense(w.q.f32, w.k.f32, w.v.f32, w.scale, rows=rows)
    assert_o(ol[:, rows], Orl, False, "wan dual local")
    assert_lse(ll[:, :, rows], Lrl, "wan dual local")
    assert_o(o[:, rows], Or, False, "wan dual full")
    assert_lse(l[:, :, rows], Lr, "wan dual full")

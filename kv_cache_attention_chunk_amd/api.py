"""PyTorch-facing binding of the chunkattn C ABI.

Argument marshalling only: tensors supply device pointers, strides and the
current HIP stream; outputs are allocated with torch when not given; every
step of the computation runs in the HIP kernels of libchunkattn.so.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import CA_BF16, CA_F32, check, lib, strides3

_DT = {torch.bfloat16: CA_BF16, torch.float32: CA_F32}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _bshd(name: str, t: torch.Tensor, dtype=torch.bfloat16):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, N, H, d]")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.numel() and t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous last dim")
    return t


def _st(t: torch.Tensor):
    """(b, n, h) element strides; an empty tensor reports contiguous ones."""
    if t.numel() == 0:
        B, N, H, d = t.shape
        return strides3((N * H * d, H * d, d))
    return strides3(t.stride()[:3])


def _i32(name: str, t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    return t


def _out(B, N, H, d, dtype, device, out):
    if out is None:
        return torch.empty((B, N, H, d), dtype=dtype, device=device)
    _bshd("out", out, dtype)
    if tuple(out.shape) != (B, N, H, d):
        raise ValueError("out has the wrong shape")
    return out


def _lse_out(B, H, N, device, lse):
    if lse is None:
        return torch.empty((B, H, N), dtype=torch.float32, device=device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    return lse


def _check_indptr(indptr, BH, Nq, q_block, q_seg):
    if indptr is None:
        return
    rows = BH * num_blocks(Nq, q_block, q_seg or max(Nq, 1))
    if indptr.numel() != rows + 1:
        raise ValueError(f"kv_indptr must have B*H*NQB + 1 = {rows + 1} entries")


_WS_BYTES = {}
_SPLIT = {True: _lib.CA_SPLIT_AUTO, "auto": _lib.CA_SPLIT_AUTO, False: _lib.CA_SPLIT_NEVER,
          "never": _lib.CA_SPLIT_NEVER, "always": _lib.CA_SPLIT_ALWAYS}


def _split(balanced) -> int:
    if balanced not in _SPLIT:
        raise ValueError("balanced must be True/'auto', False/'never' or 'always'")
    return _SPLIT[balanced]


def workspace_bytes(d: int) -> int:
    """Bytes of the balanced schedule's workspace for head dim d on the current
    device (0 when it does not apply)."""
    key = (torch.cuda.current_device(), d)
    if key not in _WS_BYTES:
        _WS_BYTES[key] = int(lib().ca_attn_workspace_bytes(d))
    return _WS_BYTES[key]


def _workspace(d: int, device, given: Optional[torch.Tensor] = None
               ) -> Tuple[Optional[torch.Tensor], int]:
    """Scratch for the balanced schedule of the dense / ragged launches: the
    caller's uint8 tensor, else one from torch's caching allocator
    (stream-ordered like every other tensor)."""
    if given is not None:
        if given.dtype != torch.uint8 or not given.is_cuda or not given.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        return given, given.numel()
    key = (torch.cuda.current_device(), d)
    if key not in _WS_BYTES:
        _WS_BYTES[key] = int(lib().ca_attn_workspace_bytes(d))
    n = _WS_BYTES[key]
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def num_blocks(n_tokens: int, block_size: int, seg_len: int) -> int:
    r = lib().ca_num_blocks(n_tokens, block_size, seg_len)
    if r < 0:
        raise ValueError("bad tiling")
    return r


def chunk_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                   kv_indptr: Optional[torch.Tensor] = None,
                   kv_indices: Optional[torch.Tensor] = None,
                   kv_block: int = 64, kv_seg: Optional[int] = None,
                   q_block: int = 64, q_seg: Optional[int] = None,
                   scale: Optional[float] = None, out_dtype=None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   o_init: Optional[torch.Tensor] = None, lse_init: Optional[torch.Tensor] = None,
                   balanced: bool = True, workspace: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk attention against a dense cache, or against per-query-block
    block lists (CSR kv_indptr / kv_indices) when given.  Returns (O, LSE).
    With (o_init float32 [B,Nq,H,d], lse_init [B,H,Nq]) from attention over a
    disjoint key set, the result is their LSE merge with this key set.
    The output dtype is out_dtype, else out's dtype, else bf16.  `balanced`
    is the key-range split policy of a dense launch: True/'auto' (split key
    ranges evenly over the device's resident workgroups when that shortens
    the launch by more than a fifth), False/'never', or 'always' (whenever it
    applies); a workspace is allocated for it unless one is given."""
    out_dtype = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    _bshd("q", q), _bshd("k", k), _bshd("v", v)
    B, Nq, H, d = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, d) or k.shape != v.shape:
        raise ValueError("k, v must be [B, Nkv, H, d] matching q")
    if k.numel() and k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    _i32("kv_indptr", kv_indptr), _i32("kv_indices", kv_indices)
    _check_indptr(kv_indptr, B * H, Nq, q_block, q_seg)
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nnz = 0 if kv_indices is None else kv_indices.numel()
    if (o_init is None) != (lse_init is None):
        raise ValueError("o_init and lse_init go together")
    if o_init is not None:
        _bshd("o_init", o_init, torch.float32)
        if tuple(o_init.shape) != (B, Nq, H, d):
            raise ValueError("o_init shape")
        if lse_init.dtype != torch.float32 or tuple(lse_init.shape) != (B, H, Nq) or \
                not lse_init.is_contiguous():
            raise ValueError("lse_init must be contiguous float32 [B, H, Nq]")
    ws, wsb = (None, 0)
    if _split(balanced) != _lib.CA_SPLIT_NEVER and kv_indptr is None and o_init is None:
        ws, wsb = _workspace(d, q.device, workspace)
    st = lib().ca_chunk_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Nq, Nkv, d,
        _st(q), _st(k), _st(o),
        _ptr(kv_indptr), _ptr(kv_indices), nnz, kv_block, kv_seg or max(Nkv, 1),
        q_block, q_seg or max(Nq, 1), sc, _ptr(o_init),
        None if o_init is None else _st(o_init), _ptr(lse_init),
        o.data_ptr(), _DT[out_dtype], l.data_ptr(), _split(balanced), _ptr(ws), wsb, _stream())
    check(st)
    return o, l


def chunk_attn_pbsa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        shared_indptr: torch.Tensor, shared_indices: torch.Tensor,
                        local_indptr: torch.Tensor, local_indices: torch.Tensor, *,
                        kv_block: int = 64, kv_seg: Optional[int] = None, q_block: int = 64,
                        q_seg: Optional[int] = None, scale: Optional[float] = None,
                        out_dtype=None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None):
    """PBSA in one pass: query block qb of head bh = b*H + h attends to the
    blocks of its head's shared list (CSR row bh: the sink and persistent
    blocks) together with its own local list (CSR row bh * NQB + qb: its
    top-K window blocks).  The two lists of a row must be disjoint; q_block
    at most 64.  Returns (O, LSE)."""
    out_dtype = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    _bshd("q", q), _bshd("k", k), _bshd("v", v)
    B, Nq, H, d = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, d) or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k, v must be [B, Nkv, H, d] matching q, with equal strides")
    for n, t in (("shared_indptr", shared_indptr), ("shared_indices", shared_indices),
                 ("local_indptr", local_indptr), ("local_indices", local_indices)):
        _i32(n, t)
    if shared_indptr.numel() != B * H + 1:
        raise ValueError("shared_indptr must have B*H + 1 entries")
    _check_indptr(local_indptr, B * H, Nq, q_block, q_seg)
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().ca_chunk_attn_pbsa_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Nq, Nkv, d, _st(q), _st(k), _st(o),
        shared_indptr.data_ptr(), shared_indices.data_ptr(), shared_indices.numel(),
        local_indptr.data_ptr(), local_indices.data_ptr(), local_indices.numel(), kv_block,
        kv_seg or max(Nkv, 1), q_block, q_seg or max(Nq, 1), sc, o.data_ptr(), _DT[out_dtype],
        l.data_ptr(), _stream())
    check(st)
    return o, l


def chunk_attn_dual_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        kv_indptr: torch.Tensor, kv_indices: torch.Tensor, local_count: int, *,
                        kv_block: int = 64, kv_seg: Optional[int] = None, q_block: int = 64,
                        q_seg: Optional[int] = None, scale: Optional[float] = None,
                        out_dtype=None, out_local: Optional[torch.Tensor] = None,
                        lse_local: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """One pass over each CSR row giving attention over the row's first
    local_count blocks (the local branch: sink + current frames) and over
    the whole row (full attention).  Returns (o_local, lse_local, o, lse);
    outputs given as out_local / lse_local / out / lse are written in place.
    The output dtype is out_dtype, else out's dtype, else bf16."""
    out_dtype = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    _bshd("q", q), _bshd("k", k), _bshd("v", v)
    B, Nq, H, d = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, d) or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k, v must be [B, Nkv, H, d] matching q, with equal strides")
    _i32("kv_indptr", kv_indptr), _i32("kv_indices", kv_indices)
    _check_indptr(kv_indptr, B * H, Nq, q_block, q_seg)
    ol = _out(B, Nq, H, d, out_dtype, q.device, out_local)
    ll = _lse_out(B, H, Nq, q.device, lse_local)
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().ca_chunk_attn_dual_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Nq, Nkv, d, _st(q), _st(k),
        kv_indptr.data_ptr(), kv_indices.data_ptr(), kv_indices.numel(), kv_block,
        kv_seg or max(Nkv, 1), q_block, q_seg or max(Nq, 1), int(local_count), sc,
        ol.data_ptr(), _st(ol), ll.data_ptr(), o.data_ptr(), _st(o), _DT[out_dtype],
        l.data_ptr(), _stream())
    check(st)
    return ol, ll, o, l


def chunk_attn_varlen_fwd(q: torch.Tensor, k_flat: torch.Tensor, v_flat: torch.Tensor,
                          cu_seqlens: torch.Tensor, *, cu_seqlens_host: Optional[np.ndarray] = None,
                          scale: Optional[float] = None, out_dtype=None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          balanced: bool = True, workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk attention against ragged per-head caches flattened into
    k_flat / v_flat [total, d] with cu_seqlens [B*H + 1] boundaries.  With
    cu_seqlens_host (a host copy equal to cu_seqlens) and `balanced`, key
    ranges are split evenly over the device's resident workgroups."""
    out_dtype = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    _bshd("q", q)
    B, Nq, H, d = q.shape
    for n, t in (("k_flat", k_flat), ("v_flat", v_flat)):
        if t.dim() != 2 or t.dtype != torch.bfloat16 or not t.is_cuda or t.shape[1] != d or \
                (t.numel() and t.stride(1) != 1):
            raise ValueError(f"{n} must be a bf16 GPU tensor [total, d]")
    if k_flat.shape != v_flat.shape or (k_flat.numel() and k_flat.stride() != v_flat.stride()):
        raise ValueError("k_flat and v_flat must match in shape and strides")
    _i32("cu_seqlens", cu_seqlens)
    if cu_seqlens.numel() != B * H + 1:
        raise ValueError("cu_seqlens must have B*H + 1 entries")
    host = None
    if cu_seqlens_host is not None:
        host = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    use = _split(balanced) != _lib.CA_SPLIT_NEVER and host is not None
    ws, wsb = _workspace(d, q.device, workspace) if use else (None, 0)
    st = lib().ca_chunk_attn_varlen_fwd(
        q.data_ptr(), k_flat.data_ptr(), v_flat.data_ptr(), cu_seqlens.data_ptr(),
        None if host is None else host.ctypes.data, k_flat.shape[0], B, H, Nq, d,
        _st(q), k_flat.stride(0) if k_flat.numel() else d, _st(o), sc,
        o.data_ptr(), _DT[out_dtype], l.data_ptr(), _split(balanced), _ptr(ws), wsb, _stream())
    check(st)
    return o, l


def chunk_attn_mixed_fwd(q: torch.Tensor, head_mode, *, k=None, v=None, kv_indptr=None,
                         kv_indices=None, kv_shared_indptr=None, kv_shared_indices=None,
                         kv_block: int = 64, kv_seg: Optional[int] = None,
                         q_block: int = 64, q_seg: Optional[int] = None, k_flat=None, v_flat=None,
                         cu_seqlens=None, cu_seqlens_host=None, scale: Optional[float] = None,
                         out_dtype=None, out=None, lse=None, balanced: bool = True,
                         workspace: Optional[torch.Tensor] = None):
    """Per-head cache modes (0 dense, 1 block lists, 2 ragged) in one call;
    dense and ragged heads share one (balanced) launch.  With
    kv_shared_indptr / kv_shared_indices (a CSR of B*H rows) the block-list
    heads run one-pass PBSA: each query block attends to its head's shared
    row together with its own kv_indptr / kv_indices row (disjoint lists,
    q_block at most 64)."""
    out_dtype = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    _bshd("q", q)
    B, Nq, H, d = q.shape
    mode = np.ascontiguousarray(head_mode, dtype=np.int32).reshape(-1)
    if mode.size != B * H:
        raise ValueError("head_mode must have B*H entries")
    Nkv = 0
    if k is not None:
        _bshd("k", k), _bshd("v", v)
        Nkv = k.shape[1]
        if k.stride() != v.stride():
            raise ValueError("k and v must share strides")
    _i32("kv_indptr", kv_indptr), _i32("kv_indices", kv_indices), _i32("cu_seqlens", cu_seqlens)
    _i32("kv_shared_indptr", kv_shared_indptr), _i32("kv_shared_indices", kv_shared_indices)
    _check_indptr(kv_indptr, B * H, Nq, q_block, q_seg)
    if kv_shared_indptr is not None and kv_shared_indptr.numel() != B * H + 1:
        raise ValueError("kv_shared_indptr must have B*H + 1 entries")
    if cu_seqlens is not None and cu_seqlens.numel() != B * H + 1:
        raise ValueError("cu_seqlens must have B*H + 1 entries")
    host = None if cu_seqlens_host is None else np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kvs = _st(k) if k is not None else strides3((0, 0, 0))
    use = _split(balanced) != _lib.CA_SPLIT_NEVER
    ws, wsb = _workspace(d, q.device, workspace) if use else (None, 0)
    st = lib().ca_chunk_attn_mixed_fwd(
        q.data_ptr(), _ptr(k), _ptr(v), B, H, Nq, Nkv, d, _st(q), kvs,
        _st(o), mode.ctypes.data, _ptr(kv_indptr), _ptr(kv_indices),
        0 if kv_indices is None else kv_indices.numel(), _ptr(kv_shared_indptr),
        _ptr(kv_shared_indices), 0 if kv_shared_indices is None else kv_shared_indices.numel(),
        kv_block, kv_seg or max(Nkv, 1),
        q_block, q_seg or max(Nq, 1), _ptr(k_flat), _ptr(v_flat), _ptr(cu_seqlens),
        None if host is None else host.ctypes.data,
        0 if k_flat is None else k_flat.shape[0], d if k_flat is None else k_flat.stride(0),
        sc, o.data_ptr(), _DT[out_dtype], l.data_ptr(), _split(balanced), _ptr(ws), wsb,
        _stream())
    check(st)
    return o, l


def lse_merge(o1: torch.Tensor, lse1: torch.Tensor, o2: torch.Tensor, lse2: torch.Tensor, *,
              out_dtype=None, out: Optional[torch.Tensor] = None,
              out_lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Recombine two attention branches over disjoint key sets via their LSE."""
    if o1.dtype != o2.dtype or o1.dtype not in _DT:
        raise TypeError("o1 and o2 must share a bf16 or float32 dtype")
    _bshd("o1", o1, o1.dtype), _bshd("o2", o2, o2.dtype)
    if o1.shape != o2.shape:
        raise ValueError("o1 and o2 shapes differ")
    B, N, H, d = o1.shape
    for n, t in (("lse1", lse1), ("lse2", lse2)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, N) or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous float32 [B, H, N]")
    od = out_dtype or (out.dtype if out is not None else o1.dtype)
    o = _out(B, N, H, d, od, o1.device, out)
    l = _lse_out(B, H, N, o1.device, out_lse)
    st = lib().ca_lse_merge(o1.data_ptr(), lse1.data_ptr(), o2.data_ptr(), lse2.data_ptr(),
                            _DT[o1.dtype], o.data_ptr(), l.data_ptr(), _DT[od], B, H, N, d,
                            _st(o1), _st(o2),
                            _st(o), _stream())
    check(st)
    return o, l


def block_mean(x: torch.Tensor, block_size: int = 64, seg_len: Optional[int] = None,
               out: Optional[torch.Tensor] = None, with_total: bool = False):
    """Block representatives: mean of each block's tokens -> float32
    [B, H, NB, d]; with_total also returns the mean over all N tokens
    [B, H, 1, d] (the chunk-mean query)."""
    _bshd("x", x)
    B, N, H, d = x.shape
    seg = seg_len or max(N, 1)
    nb = num_blocks(N, block_size, seg)
    if out is None:
        out = torch.empty((B, H, nb, d), dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, H, nb, d) or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, H, NB, d]")
    tot = torch.empty((B, H, 1, d), dtype=torch.float32, device=x.device) if with_total else None
    st = lib().ca_block_mean(x.data_ptr(), B, N, H, d, _st(x), block_size, seg,
                             out.data_ptr(), _ptr(tot), _stream())
    check(st)
    return (out, tot) if with_total else out


def block_mean_pair(x1: torch.Tensor, x2: torch.Tensor, block_size: int = 64,
                    seg_len: Optional[int] = None, with_total: bool = False):
    """block_mean of two tensors of the same shape and tiling in one launch;
    returns (means of x1, means of x2), plus x1's mean over all tokens with
    with_total."""
    _bshd("x1", x1), _bshd("x2", x2)
    if x1.shape != x2.shape:
        raise ValueError("x1 and x2 must have the same shape")
    B, N, H, d = x1.shape
    seg = seg_len or max(N, 1)
    nb = num_blocks(N, block_size, seg)
    o1 = torch.empty((B, H, nb, d), dtype=torch.float32, device=x1.device)
    o2 = torch.empty((B, H, nb, d), dtype=torch.float32, device=x1.device)
    tot = torch.empty((B, H, 1, d), dtype=torch.float32, device=x1.device) if with_total else None
    st = lib().ca_block_mean_pair(x1.data_ptr(), _st(x1), o1.data_ptr(), _ptr(tot), x2.data_ptr(),
                                  _st(x2), o2.data_ptr(), B, N, H, d, block_size, seg, _stream())
    check(st)
    return (o1, o2, tot) if with_total else (o1, o2)


def block_score_topk(q_mean: torch.Tensor, k_mean: torch.Tensor, K: int, *, cand_begin: int = 0,
                     cand_count: Optional[int] = None, return_scores: bool = False):
    """Top-K candidate blocks per query block by representative dot product;
    ids ascending, ties toward the lower id."""
    for n, t in (("q_mean", q_mean), ("k_mean", k_mean)):
        if t.dtype != torch.float32 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 GPU tensor [B, H, N, d]")
    B, H, NQB, d = q_mean.shape
    NKB = k_mean.shape[2]
    if tuple(k_mean.shape) != (B, H, NKB, d):
        raise ValueError("k_mean shape mismatch")
    cc = NKB - cand_begin if cand_count is None else cand_count
    idx = torch.empty((B, H, NQB, K), dtype=torch.int32, device=q_mean.device)
    sc = torch.empty((B, H, NQB, K), dtype=torch.float32, device=q_mean.device) if return_scores else None
    st = lib().ca_block_score_topk(q_mean.data_ptr(), k_mean.data_ptr(), B, H, NQB, NKB, d,
                                   cand_begin, cc, K, idx.data_ptr(), _ptr(sc), _stream())
    check(st)
    return (idx, sc) if return_scores else idx


def block_score_topk_lists(q_mean: torch.Tensor, k_mean: torch.Tensor, K: int, *,
                           cand_begin: int = 0, cand_count: Optional[int] = None,
                           prefix_begin: int = 0, prefix_count: int = 0, id_offset: int = 0):
    """block_score_topk that also returns the PBSA block lists of the selection
    (one launch): CSR row (b, h, qb) = prefix_begin .. prefix_begin +
    prefix_count - 1, then id_offset + the K selected ids.  The prefix must lie
    below every selected id + id_offset.  Returns (idx, indptr, indices)."""
    for n, t in (("q_mean", q_mean), ("k_mean", k_mean)):
        if t.dtype != torch.float32 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 GPU tensor [B, H, N, d]")
    B, H, NQB, d = q_mean.shape
    NKB = k_mean.shape[2]
    if tuple(k_mean.shape) != (B, H, NKB, d):
        raise ValueError("k_mean shape mismatch")
    cc = NKB - cand_begin if cand_count is None else cand_count
    rows = B * H * NQB
    dev = q_mean.device
    idx = torch.empty((B, H, NQB, K), dtype=torch.int32, device=dev)
    indptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    indices = torch.empty(max(rows * (prefix_count + K), 1), dtype=torch.int32, device=dev)
    st = lib().ca_block_score_topk_lists(q_mean.data_ptr(), k_mean.data_ptr(), B, H, NQB, NKB, d,
                                         cand_begin, cc, K, prefix_begin, prefix_count, id_offset,
                                         idx.data_ptr(), indptr.data_ptr(), indices.data_ptr(),
                                         _stream())
    check(st)
    return idx, indptr, indices


def block_score_topk_batch(jobs):
    """Up to four independent selections in one launch.  Each job is a dict
    with q_mean, k_mean, K and optionally cand_begin, cand_count and, for
    block lists, prefix_begin, prefix_count, id_offset and lists=True.
    Returns one result per job: idx, or (idx, indptr, indices) with lists."""
    from ._lib import TopkJob
    if not 1 <= len(jobs) <= 4:
        raise ValueError("1 to 4 jobs")
    arr = (TopkJob * len(jobs))()
    res, keep = [], []
    for n, jb in enumerate(jobs):
        qm, km, K = jb["q_mean"], jb["k_mean"], jb["K"]
        for name, t in (("q_mean", qm), ("k_mean", km)):
            if t.dtype != torch.float32 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 GPU tensor [B, H, N, d]")
        B, H, NQB, d = qm.shape
        NKB = km.shape[2]
        if tuple(km.shape) != (B, H, NKB, d):
            raise ValueError("k_mean shape mismatch")
        cb = jb.get("cand_begin", 0)
        cc = jb.get("cand_count", NKB - cb)
        idx = torch.empty((B, H, NQB, K), dtype=torch.int32, device=qm.device)
        ip = ix = None
        pb, pc, off = jb.get("prefix_begin", 0), jb.get("prefix_count", 0), jb.get("id_offset", 0)
        if jb.get("lists"):
            rows = B * H * NQB
            ip = torch.empty(rows + 1, dtype=torch.int32, device=qm.device)
            ix = torch.empty(max(rows * (pc + K), 1), dtype=torch.int32, device=qm.device)
        arr[n] = TopkJob(qm.data_ptr(), km.data_ptr(), B, H, NQB, NKB, d, cb, cc, K, pb, pc, off,
                         idx.data_ptr(), None, _ptr(ip), _ptr(ix))
        res.append((idx, ip, ix) if ip is not None else idx)
        keep += [qm, km]
    check(lib().ca_block_score_topk_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream()))
    return res


def persistent_update(q_mean: torch.Tensor, k_mean: torch.Tensor,
                      persistent: Optional[torch.Tensor], evict_begin: int, evict_count: int,
                      C: int, *, out: Optional[torch.Tensor] = None, return_scores: bool = False):
    """New persistent block set per head when the local window slides: the
    top C of (current persistent ids) U (evicted blocks [evict_begin,
    evict_begin + evict_count)) by <q_mean, k_mean[id]>, ids ascending, -1
    padding.  `out` may be `persistent` itself (in-place update)."""
    for n, t in (("q_mean", q_mean), ("k_mean", k_mean)):
        if t.dtype != torch.float32 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 GPU tensor [B, H, N, d]")
    B, H, one, d = q_mean.shape
    NKB = k_mean.shape[2]
    if one != 1 or tuple(k_mean.shape) != (B, H, NKB, d):
        raise ValueError("q_mean must be [B, H, 1, d] and k_mean [B, H, NKB, d]")
    C_in = 0
    if persistent is not None:
        _i32("persistent", persistent)
        if persistent.dim() != 3 or tuple(persistent.shape[:2]) != (B, H):
            raise ValueError("persistent must be [B, H, C_in]")
        C_in = persistent.shape[2]
    if out is None:
        out = torch.empty((B, H, C), dtype=torch.int32, device=q_mean.device)
    else:
        _i32("out", out)
        if tuple(out.shape) != (B, H, C):
            raise ValueError("out must be [B, H, C]")
    sc = torch.empty((B, H, C), dtype=torch.float32, device=q_mean.device) if return_scores else None
    st = lib().ca_persistent_update(q_mean.data_ptr(), k_mean.data_ptr(), B, H, NKB, d,
                                    _ptr(persistent), C_in, evict_begin, evict_count, C,
                                    out.data_ptr(), _ptr(sc), _stream())
    check(st)
    return (out, sc) if return_scores else out


def pack_plan(frames, device) -> dict:
    """Device-side frame lists for pack_ragged: frames[bh] lists head bh's
    output frames in order; an entry is a source frame id (copied) or a pair
    (a, b) of frames merged into one."""
    ptr = np.zeros(len(frames) + 1, np.int32)
    src = []
    for bh, fl in enumerate(frames):
        for f in fl:
            a, b = (int(f[0]), int(f[1])) if isinstance(f, (tuple, list)) else (int(f), -1)
            src.append((a, b))
        ptr[bh + 1] = len(src)
    F = len(src)
    src_np = np.array(src, np.int32).reshape(-1) if F else np.zeros(2, np.int32)
    return {"heads": len(frames), "frames": F, "ptr_host": ptr,
            "ptr": torch.from_numpy(ptr).to(device), "src": torch.from_numpy(src_np).to(device)}


def pack_ragged(k: torch.Tensor, v: torch.Tensor, frames, frame_tokens: int, *,
                out_k: Optional[torch.Tensor] = None, out_v: Optional[torch.Tensor] = None,
                out_cu: Optional[torch.Tensor] = None):
    """Flatten per-head frame selections of a dense cache k, v [B, N, H, d]
    into k_flat, v_flat [sum of frames * frame_tokens, d] + cu_seqlens.
    `frames` is a list per head (see pack_plan) or a plan from pack_plan.
    Merged frames are the float32 average rounded to bf16.  Returns (k_flat,
    v_flat, cu_seqlens, cu_seqlens_host); out_k / out_v (contiguous bf16
    [rows, d]) and out_cu (int32 [B*H + 1]) are written in place when given."""
    _bshd("k", k), _bshd("v", v)
    B, N, H, d = k.shape
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must match in shape and strides")
    plan = frames if isinstance(frames, dict) else pack_plan(frames, k.device)
    if plan["heads"] != B * H:
        raise ValueError("frames must list B*H heads")
    F = plan["frames"]

    def flat_out(name, t):
        if t is None:
            return torch.empty((F * frame_tokens, d), dtype=torch.bfloat16, device=k.device)
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or \
                tuple(t.shape) != (F * frame_tokens, d):
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [{F * frame_tokens}, {d}]")
        return t
    kf, vf = flat_out("out_k", out_k), flat_out("out_v", out_v)
    if out_cu is None:
        cu = torch.empty(B * H + 1, dtype=torch.int32, device=k.device)
    else:
        cu = _i32("out_cu", out_cu)
        if cu.numel() != B * H + 1:
            raise ValueError("out_cu must have B*H + 1 entries")
    st = lib().ca_pack_ragged(k.data_ptr(), v.data_ptr(), B, N, H, d, _st(k), frame_tokens,
                              plan["ptr"].data_ptr(), plan["ptr_host"].ctypes.data, F,
                              plan["src"].data_ptr(), kf.data_ptr(), vf.data_ptr(), d,
                              cu.data_ptr(), _stream())
    check(st)
    return kf, vf, cu, plan["ptr_host"] * frame_tokens


def cast_bf16_to_f16(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16 copy (round to nearest even) of a contiguous bf16 GPU tensor."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 GPU tensor")
    y = torch.empty(x.shape, dtype=torch.float16, device=x.device) if out is None else out
    check(lib().ca_cast_bf16_to_f16(x.data_ptr(), y.data_ptr(), x.numel(), _stream()))
    return y


def mla_chunk_attn(q: torch.Tensor, kv_lat: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                   *, scale: Optional[float] = None, out_dtype=torch.bfloat16,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   o_lat: Optional[torch.Tensor] = None):
    """Chunk attention over a latent KV cache (d_c = 192, d_rope = 32):
    q bf16 [B, Nq, H, 128] (content 96 + position 32), kv_lat fp16
    [B, N, 224] (rows [c ; k^R]), w_uk bf16 [H, 96, 192], w_uv bf16
    [H, 128, 192].  Absorbs W^K into the queries (fp16, with the rounding
    residual kept for the LSE's first-order correction), attends every
    (query, head) row to the latent rows, projects with W^V.  Returns
    (o, lse, o_lat);
    outputs given as out / lse / o_lat (float32 [B, Nq, H, 192],
    contiguous) are written in place."""
    _bshd("q", q)
    B, Nq, H, dq = q.shape
    if kv_lat.dtype != torch.float16 or kv_lat.dim() != 3 or kv_lat.shape[0] != B or \
            kv_lat.shape[2] != 224 or kv_lat.stride(2) != 1:
        raise ValueError("kv_lat must be fp16 [B, N, 224] with contiguous rows")
    for n, w, shp in (("w_uk", w_uk, (H, 96, 192)), ("w_uv", w_uv, (H, 128, 192))):
        if w.dtype != torch.bfloat16 or tuple(w.shape) != shp or not w.is_contiguous():
            raise ValueError(f"{n} must be a contiguous bf16 tensor {shp}")
    N = kv_lat.shape[1]
    sc = 1.0 / math.sqrt(dq) if scale is None else float(scale)
    q_lat = torch.empty((B, Nq, H, 224), dtype=torch.float16, device=q.device)
    q_lo = torch.empty((B, Nq, H, 192), dtype=torch.bfloat16, device=q.device)
    check(lib().ca_mla_absorb_q(q.data_ptr(), B, Nq, H, 96, dq - 96, 192, _st(q), w_uk.data_ptr(),
                                q_lat.data_ptr(), q_lo.data_ptr(), _stream()))
    if o_lat is None:
        o_lat = torch.empty((B, Nq, H, 192), dtype=torch.float32, device=q.device)
    elif o_lat.dtype != torch.float32 or tuple(o_lat.shape) != (B, Nq, H, 192) or \
            not o_lat.is_contiguous() or not o_lat.is_cuda:
        raise ValueError("o_lat must be a contiguous float32 GPU tensor [B, Nq, H, 192]")
    lse = _lse_out(B, H, Nq, q.device, lse)
    check(lib().ca_mla_attn_fwd(q_lat.data_ptr(), q_lo.data_ptr(), kv_lat.data_ptr(), B, Nq, H, N,
                                192, 32,
                                kv_lat.stride(0) if N else 0, kv_lat.stride(1) if N else 224, sc,
                                o_lat.data_ptr(), lse.data_ptr(), _stream()))
    o = _out(B, Nq, H, 128, out_dtype, q.device, out)
    check(lib().ca_mla_up_proj(o_lat.data_ptr(), w_uv.data_ptr(), B, Nq, H, 192, 128, o.data_ptr(),
                               _DT[out_dtype], _st(o), _stream()))
    return o, lse, o_lat


def build_kv_index(B: int, H: int, NQB: int, sink_begin: int, sink_count: int,
                   persistent: Optional[torch.Tensor], topk: Optional[torch.Tensor],
                   topk_offset: int = 0, device=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """PBSA block lists: CSR rows = sorted union of sink, persistent, top-K."""
    C = 0 if persistent is None else persistent.shape[-1]
    K = 0 if topk is None else topk.shape[-1]
    _i32("persistent", persistent), _i32("topk", topk)
    dev = device or (persistent.device if persistent is not None else topk.device)
    rows = B * H * NQB
    indptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    indices = torch.empty(max(rows * (sink_count + C + K), 1), dtype=torch.int32, device=dev)
    st = lib().ca_build_kv_index(B, H, NQB, sink_begin, sink_count, _ptr(persistent), C, _ptr(topk),
                                 K, topk_offset, indptr.data_ptr(), indices.data_ptr(), _stream())
    check(st)
    return indptr, indices


def block_sparse_workspace(B: int, H: int, Nq: int, Nkv: int, d: int, *, block: int, seg: int,
                           sink_begin: int, sink_count: int, hist_begin: int, hist_count: int,
                           C: int, local_begin: int, local_count: int, K: int,
                           have_k_mean: bool) -> "_lib.BlockSparseWs":
    """Workspace layout of block_sparse_fwd (sizes and byte offsets)."""
    layout = _lib.BlockSparseWs()
    n = lib().ca_block_sparse_workspace(B, H, Nq, Nkv, d, block, seg, sink_begin, sink_count,
                                        hist_begin, hist_count, C, local_begin, local_count, K,
                                        int(bool(have_k_mean)), ctypes.byref(layout))
    if n == 0:
        check(_lib.CA_EINVAL)
    return layout


def block_sparse_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, sink_begin: int,
                     sink_count: int, hist_begin: int, hist_count: int, C: int,
                     local_begin: int, local_count: int, K: int, block: int = 64,
                     seg: Optional[int] = None, k_mean: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, out_dtype=torch.bfloat16,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """The block-sparse path in the Sparse Forcing order, one native call
    (ca_block_sparse_fwd): block means of Q and K (and the chunk-mean query),
    persistent blocks = top-C history blocks against the chunk-mean query,
    top-K local-window blocks per query block, then PBSA in one pass: every
    query block attends to the blocks its head shares (sink + persistent)
    together with its own top-K local blocks.  The sink, history and local
    id ranges must be disjoint.

    `k_mean` carries key-block means of the cache kept from earlier steps
    (resident state, [B, H, NB, d] float32); only the history entries are
    read from it, and the local window's means are recomputed from k.
    Returns (O, LSE, info); `info` holds views into the workspace: the block
    means, the selected ids and the block lists (info["local"] holds ids
    relative to info["local_base"])."""
    out_dtype = out.dtype if out is not None else out_dtype
    _bshd("q", q), _bshd("k", k), _bshd("v", v)
    B, Nq, H, d = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, d) or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k, v must be [B, Nkv, H, d] matching q, with equal strides")
    seg = seg or Nq
    nkb, nqb = num_blocks(Nkv, block, seg), num_blocks(Nq, block, seg)
    if k_mean is not None:
        if k_mean.dtype != torch.float32 or tuple(k_mean.shape) != (B, H, nkb, d) or \
                not k_mean.is_contiguous() or not k_mean.is_cuda:
            raise ValueError(f"k_mean must be a contiguous float32 GPU tensor [B, H, {nkb}, d]")
    ranges = dict(sink_begin=sink_begin, sink_count=sink_count, hist_begin=hist_begin,
                  hist_count=hist_count, C=C, local_begin=local_begin, local_count=local_count, K=K)
    lay = block_sparse_workspace(B, H, Nq, Nkv, d, block=block, seg=seg,
                                 have_k_mean=k_mean is not None, **ranges)
    if workspace is None:
        workspace = torch.empty(lay.bytes, dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    o = _out(B, Nq, H, d, out_dtype, q.device, out)
    l = _lse_out(B, H, Nq, q.device, lse)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().ca_block_sparse_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Nq, Nkv, d, _st(q), _st(k), _st(o), block,
        seg, sink_begin, sink_count, hist_begin, hist_count, C, local_begin, local_count, K,
        _ptr(k_mean), sc, o.data_ptr(), _DT[out_dtype], l.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream())
    check(st)

    def view(off, dtype, shape):
        n = int(np.prod(shape))
        size = torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + n * size].view(dtype).view(*shape)
    f32, i32t = torch.float32, torch.int32
    km = view(lay.k_mean, f32, (B, H, nkb, d)) if lay.k_mean_in_ws else k_mean
    km_loc = view(lay.k_mean_local, f32, (B, H, local_count, d)) if lay.window_means else km
    info = {"q_mean": view(lay.q_mean, f32, (B, H, nqb, d)), "k_mean": km,
            "k_mean_local": km_loc, "chunk_mean": view(lay.chunk_mean, f32, (B, H, 1, d)),
            "persistent": view(lay.persistent, i32t, (B, H, 1, C)) if C else None,
            "local": view(lay.local, i32t, (B, H, nqb, K)) if K else None,
            "local_base": int(lay.local_id_base),
            "shared_indptr": view(lay.shared_indptr, i32t, (B * H + 1,)),
            "shared_indices": view(lay.shared_indices, i32t, (B * H * (sink_count + C),)),
            "local_indptr": view(lay.local_indptr, i32t, (B * H * nqb + 1,)),
            "local_indices": view(lay.local_indices, i32t, (B * H * nqb * K,)),
            "workspace": workspace}
    return o, l, info

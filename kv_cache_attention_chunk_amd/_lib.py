"""ctypes declarations of the libchunkattn.so C ABI (include/chunkattn.h).

The library is loaded on first use from this package's directory.  A missing
library is an error: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libchunkattn.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "chunkattn.h")

ABI_VERSION = 4
CA_OK, CA_EINVAL, CA_EUNSUPPORTED, CA_ERANGE, CA_ENODEV, CA_EHIP = range(6)
CA_BF16, CA_F32 = 0, 1
CA_MODE_DENSE, CA_MODE_BLOCKS, CA_MODE_VARLEN = 0, 1, 2
CA_SPLIT_AUTO, CA_SPLIT_NEVER, CA_SPLIT_ALWAYS = 0, 1, 2
CA_SCRATCH_BYTES = 16 << 20     # device scratch of ca_block_sparse_fwd_noalloc, per GPU

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_i64 = ctypes.c_int64
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.c_void_p   # device or host int32 pointers are passed as addresses
_sz = ctypes.c_size_t

SIGNATURES = {
    "ca_abi_version": (_i, []),
    "ca_status_str": (ctypes.c_char_p, [_i]),
    "ca_last_error": (ctypes.c_char_p, []),
    "ca_num_blocks": (_i, [_i, _i, _i]),
    "ca_attn_workspace_bytes": (_sz, [_i]),
    "ca_chunk_attn_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i64p,
                               _i32p, _i32p, _i, _i, _i, _i, _i, _f, _p, _i64p, _p,
                               _p, _i, _p, _i, _p, _sz, _p]),
    "ca_chunk_attn_dual_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i32p, _i32p,
                                    _i, _i, _i, _i, _i, _i, _f, _p, _i64p, _p, _p, _i64p, _i,
                                    _p, _p]),
    "ca_chunk_attn_pbsa_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i64p,
                                    _i32p, _i32p, _i, _i32p, _i32p, _i, _i, _i, _i, _i, _f,
                                    _p, _i, _p, _p]),
    "ca_block_sparse_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                        _i, _i, _p]),
    "ca_block_sparse_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i64p, _i, _i,
                                 _i, _i, _i, _i, _i, _i, _i, _i, _p, _f, _p, _i, _p, _p, _sz,
                                 _p]),
    "ca_block_sparse_fwd_noalloc": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i64p,
                                         _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _f, _p, _i,
                                         _p, _p]),
    "ca_chunk_attn_varlen_fwd": (_i, [_p, _p, _p, _i32p, _i32p, _i, _i, _i, _i, _i,
                                      _i64p, _i64, _i64p, _f, _p, _i, _p, _i, _p, _sz, _p]),
    "ca_chunk_attn_mixed_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i64p, _i64p, _i64p,
                                     _i32p, _i32p, _i32p, _i, _i32p, _i32p, _i, _i, _i, _i, _i,
                                     _p, _p,
                                     _i32p, _i32p, _i, _i64, _f, _p, _i, _p, _i, _p, _sz, _p]),
    "ca_lse_merge": (_i, [_p, _p, _p, _p, _i, _p, _p, _i, _i, _i, _i, _i,
                          _i64p, _i64p, _i64p, _p]),
    "ca_block_mean": (_i, [_p, _i, _i, _i, _i, _i64p, _i, _i, _p, _p, _p]),
    "ca_block_mean_pair": (_i, [_p, _i64p, _p, _p, _p, _i64p, _p, _i, _i, _i, _i, _i, _i, _p]),
    "ca_block_score_topk": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "ca_block_score_topk_lists": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                       _p, _p, _p, _p]),
    "ca_block_score_topk_batch": (_i, [_p, _i, _p]),
    "ca_persistent_update": (_i, [_p, _p, _i, _i, _i, _i, _i32p, _i, _i, _i, _i, _p, _p, _p]),
    "ca_pack_ragged": (_i, [_p, _p, _i, _i, _i, _i, _i64p, _i, _i32p, _i32p, _i, _i32p, _p, _p,
                            _i64, _p, _p]),
    "ca_mla_absorb_q": (_i, [_p, _i, _i, _i, _i, _i, _i, _i64p, _p, _p, _p, _p]),
    "ca_mla_attn_fwd": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _f, _p, _p, _p]),
    "ca_mla_up_proj": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _i, _i64p, _p]),
    "ca_cast_bf16_to_f16": (_i, [_p, _p, _i64, _p]),
    "ca_build_kv_index": (_i, [_i, _i, _i, _i, _i, _i32p, _i, _i32p, _i, _i, _p, _p, _p]),
}

_LIB = None


class TopkJob(ctypes.Structure):
    """ctypes mirror of ca_topk_job (include/chunkattn.h)."""
    _fields_ = [("q_mean", ctypes.c_void_p), ("k_mean", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("NQB", ctypes.c_int),
                ("NKB", ctypes.c_int), ("d", ctypes.c_int),
                ("cand_begin", ctypes.c_int), ("cand_count", ctypes.c_int), ("K", ctypes.c_int),
                ("prefix_begin", ctypes.c_int), ("prefix_count", ctypes.c_int),
                ("id_offset", ctypes.c_int),
                ("out_idx", ctypes.c_void_p), ("out_score", ctypes.c_void_p),
                ("indptr", ctypes.c_void_p), ("indices", ctypes.c_void_p)]


class BlockSparseWs(ctypes.Structure):
    """ctypes mirror of ca_block_sparse_ws (include/chunkattn.h)."""
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "bytes", "q_mean", "k_mean", "k_mean_local", "chunk_mean", "persistent", "local",
        "shared_indptr", "shared_indices", "local_indptr", "local_indices")] + \
        [(n, ctypes.c_int) for n in ("window_means", "window_token0", "window_tokens",
                                     "local_id_base", "k_mean_in_ws")]


def header_functions():
    """Names of the functions include/chunkattn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_\w+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m kv_cache_attention_chunk_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.ca_abi_version() != ABI_VERSION:
            raise RuntimeError("libchunkattn ABI version mismatch")
        _LIB = L
    return _LIB


class ChunkAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def check(status: int) -> None:
    if status == CA_OK:
        return
    msg = lib().ca_last_error().decode(errors="replace")
    if status in (CA_EINVAL, CA_ERANGE):
        raise ValueError(f"chunkattn: {msg} (status {status})")
    if status == CA_EUNSUPPORTED:
        raise NotImplementedError(f"chunkattn: {msg}")
    raise ChunkAttnError(status, f"chunkattn: {msg}")


def strides3(s) -> ctypes.Array:
    return (ctypes.c_int64 * 3)(*[int(x) for x in s])

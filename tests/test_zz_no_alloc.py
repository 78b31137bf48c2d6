"""The allocation-free block-sparse call (ca_block_sparse_fwd_noalloc, for
callers that cannot allocate device memory) against the workspace call
(ca_block_sparse_fwd), both through the C ABI: two calls in a row, the
second on a smaller input, must give outputs bit-identical to the workspace
call's on the same inputs (the same kernels run on the library's own
scratch).  Sizes beyond the scratch are rejected before any launch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
from kv_cache_attention_chunk_amd import _lib
from kv_cache_attention_chunk_amd import workloads as wl
from kv_cache_attention_chunk_amd._lib import CA_BF16, CA_ERANGE, CA_OK, strides3

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(t):
    return torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _args(q, k, v, lay, k_mean, scale, o, l):
    B, Nq, H, d = q.shape
    return [q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Nq, k.shape[1], d,
            strides3(q.stride()[:3]), strides3(k.stride()[:3]), strides3(o.stride()[:3]), 64,
            lay["seg"], 0, lay["sink_count"], lay["hist_begin"], lay["hist_count"], lay["C"],
            lay["local_begin"], lay["local_count"], lay["K"],
            None if k_mean is None else k_mean.data_ptr(), scale, o.data_ptr(), CA_BF16,
            l.data_ptr()]


def _case(seed, H, frames_q, frames_kv, ratio, resident):
    w = wl.wan_dense(seed=seed, H=H, frames_q=frames_q, frames_kv=frames_kv)
    lay = dict(wl.sparse_layout(w, ratio), seg=1560)
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    km = ca.block_mean(k, 64, 1560) if resident else None
    return w, lay, q, k, v, km


def test_noalloc_matches_the_workspace_call_twice():
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    cases = [("Wan layer, 12 heads, resident key means, K = 10", (0, 12, 3, 21, 0.125, True)),
             ("smaller: 5 heads, 2-frame chunk, 9-frame cache, no resident means, K = 13",
              (3, 5, 2, 9, 0.25, False))]
    for what, spec in cases:
        say(f"no-alloc block-sparse: {what}")
        w, lay, q, k, v, km = _case(*spec)
        B, Nq, H, d = q.shape
        o_ws = torch.full_like(q, float("nan"))
        l_ws = torch.full((B, H, Nq), float("nan"), device="cuda")
        n = L.ca_block_sparse_workspace(B, H, Nq, k.shape[1], d, 64, 1560, 0, lay["sink_count"],
                                        lay["hist_begin"], lay["hist_count"], lay["C"],
                                        lay["local_begin"], lay["local_count"], lay["K"],
                                        int(km is not None), None)
        assert 0 < n <= _lib.CA_SCRATCH_BYTES
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        st = L.ca_block_sparse_fwd(*_args(q, k, v, lay, km, w.scale, o_ws, l_ws), ws.data_ptr(),
                                   n, stream)
        assert st == CA_OK, L.ca_last_error()
        o_na = torch.full_like(q, float("nan"))
        l_na = torch.full((B, H, Nq), float("nan"), device="cuda")
        st = L.ca_block_sparse_fwd_noalloc(*_args(q, k, v, lay, km, w.scale, o_na, l_na), stream)
        assert st == CA_OK, L.ca_last_error()
        torch.cuda.synchronize()
        assert not torch.isnan(o_na.float()).any() and not torch.isnan(l_na).any()
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), what
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), what


def test_noalloc_rejects_sizes_beyond_its_scratch():
    L = _lib.lib()
    # 64 heads of the Wan layer without resident key means: about 22 MB of
    # intermediates, above the 16 MiB the library holds
    B, H, Nq, Nkv, d = 1, 64, 4680, 32760, 128
    need = L.ca_block_sparse_workspace(B, H, Nq, Nkv, d, 64, 1560, 0, 25, 25, 425, 32, 450, 75,
                                       10, 0, None)
    assert need > _lib.CA_SCRATCH_BYTES
    x = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")   # never read
    S = strides3((Nq * H * d, H * d, d))
    Skv = strides3((Nkv * H * d, H * d, d))
    st = L.ca_block_sparse_fwd_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), B, H, Nq, Nkv, d,
                                       S, Skv, S, 64, 1560, 0, 25, 25, 425, 32, 450, 75, 10, None,
                                       0.088, x.data_ptr(), CA_BF16, x.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == CA_ERANGE and b"scratch" in L.ca_last_error()

"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before touching a device (CPU only)."""
import ctypes

import numpy as np
import pytest
import torch

from kv_cache_attention_chunk_amd import _lib
from kv_cache_attention_chunk_amd._lib import (CA_EINVAL, CA_ENODEV, CA_ERANGE, CA_EUNSUPPORTED,
                                               strides3)

FAKE = 0x10000          # 16-byte aligned dummy address; never dereferenced
S = strides3((4680 * 12 * 128, 12 * 128, 128))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _lib.header_functions()
    assert len(names) == 26
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_header_constants_match_the_binding():
    text = open(_lib.HEADER).read()
    assert f"#define CA_ABI_VERSION {_lib.ABI_VERSION}" in text
    assert "#define CA_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert _lib.CA_SCRATCH_BYTES == 16 << 20


def test_status_strings_and_version(L):
    assert L.ca_abi_version() == 4
    for code, word in [(0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"range"),
                       (4, b"device"), (5, b"HIP")]:
        assert word in L.ca_status_str(code)


def test_num_blocks(L):
    assert L.ca_num_blocks(32760, 64, 1560) == 525
    assert L.ca_num_blocks(4680, 64, 1560) == 75
    assert L.ca_num_blocks(1024, 64, 1024) == 16
    assert L.ca_num_blocks(100, 64, 60) == 2
    assert L.ca_num_blocks(0, 64, 1560) == 0
    assert L.ca_num_blocks(10, 0, 5) == -1


def fwd(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, H=12, Nq=4680, Nkv=32760, d=128, qs=S, kvs=S, os=S,
             indptr=None, indices=None, nnz=0, kb=64, ks=1560, qb=64, qseg=1560, scale=0.088,
             oi=None, ois=None, li=None, o=FAKE, odt=0, lse=FAKE, split=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return L.ca_chunk_attn_fwd(a["q"], a["k"], a["v"], a["B"], a["H"], a["Nq"], a["Nkv"], a["d"],
                               a["qs"], a["kvs"], a["os"], a["indptr"], a["indices"], a["nnz"],
                               a["kb"], a["ks"], a["qb"], a["qseg"], a["scale"], a["oi"], a["ois"],
                               a["li"], a["o"], a["odt"], a["lse"], a["split"], a["ws"], a["wsb"],
                               a["stream"])


def test_attention_argument_errors(L):
    assert fwd(L, q=None) == CA_EINVAL
    assert fwd(L, q=FAKE + 8) == CA_EINVAL
    assert fwd(L, d=96) == CA_EUNSUPPORTED
    assert fwd(L, odt=7) == CA_EUNSUPPORTED
    assert fwd(L, B=-1) == CA_EINVAL
    assert fwd(L, qs=strides3((1, 3, 128))) == CA_EINVAL
    assert fwd(L, indptr=FAKE) == CA_EINVAL                 # indices missing
    assert fwd(L, indptr=FAKE, indices=FAKE, kb=65) == CA_ERANGE
    assert fwd(L, indptr=FAKE, indices=FAKE, nnz=-1) == CA_EINVAL
    assert fwd(L, scale=float("nan")) == CA_EINVAL
    assert fwd(L, scale=-0.1) == CA_EINVAL
    assert fwd(L, oi=FAKE, ois=S) == CA_EINVAL                 # lse_init missing
    assert fwd(L, oi=FAKE, ois=S, li=FAKE, o=FAKE, odt=0) == CA_EINVAL   # aliases o_init as bf16
    assert fwd(L, kvs=strides3((0, 64, 8))) == CA_ERANGE        # row stride below d
    assert fwd(L, ws=FAKE + 8, wsb=1 << 20) == CA_EINVAL         # misaligned workspace
    assert fwd(L, ws=None, wsb=1 << 20) == CA_EINVAL             # size without a workspace
    assert fwd(L, split=3) == CA_EINVAL                          # unknown split policy
    fwd(L, d=96)
    assert b"head dim 96" in L.ca_last_error()


def pbsa(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, H=12, Nq=4680, Nkv=32760, d=128, qs=S, kvs=S, os=S,
             sp=FAKE, si=FAKE, sn=684, lp=FAKE, li=FAKE, ln=9000, kb=64, ks=1560, qb=64,
             qseg=1560, scale=0.088, o=FAKE, odt=0, lse=FAKE, stream=None)
    a.update(kw)
    return L.ca_chunk_attn_pbsa_fwd(a["q"], a["k"], a["v"], a["B"], a["H"], a["Nq"], a["Nkv"],
                                    a["d"], a["qs"], a["kvs"], a["os"], a["sp"], a["si"], a["sn"],
                                    a["lp"], a["li"], a["ln"], a["kb"], a["ks"], a["qb"],
                                    a["qseg"], a["scale"], a["o"], a["odt"], a["lse"],
                                    a["stream"])


def test_pbsa_argument_errors(L):
    assert pbsa(L, sp=None) == CA_EINVAL                 # shared list missing
    assert pbsa(L, li=None) == CA_EINVAL                 # local indices missing
    assert pbsa(L, qb=65) == CA_ERANGE                   # a query block above 64 rows
    assert b"q_block" in L.ca_last_error()
    assert pbsa(L, kb=65) == CA_ERANGE
    assert pbsa(L, ln=-1) == CA_EINVAL
    assert pbsa(L, d=80) == CA_EUNSUPPORTED
    assert pbsa(L, k=FAKE + 4) == CA_EINVAL
    assert pbsa(L, scale=0.0) == CA_EINVAL


def test_block_sparse_workspace_layout(L):
    """Workspace sizes and offsets of the block-sparse pipeline at the Wan
    shape: query-block means, window means (resident history means) or every
    key block's means, ids and lists, each 256-byte aligned and disjoint."""
    ws = _lib.BlockSparseWs()
    args = (1, 12, 4680, 32760, 128, 64, 1560, 0, 25, 25, 425, 32, 450, 75, 10)
    n = L.ca_block_sparse_workspace(*args, 1, ctypes.byref(ws))
    assert n == ws.bytes > 0
    assert ws.window_means == 1 and ws.window_token0 == 18 * 1560 and ws.window_tokens == 4680
    assert ws.local_id_base == 450 and ws.k_mean_in_ws == 0
    offs = [ws.q_mean, ws.k_mean_local, ws.chunk_mean, ws.persistent, ws.local,
            ws.shared_indptr, ws.shared_indices, ws.local_indptr, ws.local_indices]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert ws.k_mean_local - ws.q_mean >= 12 * 75 * 128 * 4
    assert ws.bytes < (2 << 20)                    # about 1 MB at this shape
    ws2 = _lib.BlockSparseWs()
    n2 = L.ca_block_sparse_workspace(*args, 0, ctypes.byref(ws2))
    assert ws2.k_mean_in_ws == 1 and ws2.window_means == 0 and ws2.local_id_base == 0
    assert n2 - n >= 12 * 525 * 128 * 4 - 12 * 75 * 128 * 4
    # overlapping ranges, K above the window, block above 64: rejected
    bad = list(args)
    bad[10] = 430                                  # history overlaps the local window
    assert L.ca_block_sparse_workspace(*bad, 1, None) == 0
    assert b"disjoint" in L.ca_last_error()
    bad = list(args)
    bad[14] = 76
    assert L.ca_block_sparse_workspace(*bad, 1, None) == 0
    bad = list(args)
    bad[5] = 65
    assert L.ca_block_sparse_workspace(*bad, 1, None) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is visible")
def test_no_device_reports_enodev(L):
    assert fwd(L) == CA_ENODEV
    assert fwd(L, indptr=FAKE, indices=FAKE, nnz=10) == CA_ENODEV
    assert b"no HIP device" in L.ca_last_error()


def test_varlen_host_checks(L):
    cu = np.array([0, 10, 5], dtype=np.int32)
    st = L.ca_chunk_attn_varlen_fwd(FAKE, FAKE, FAKE, FAKE, cu.ctypes.data, 100, 1, 2, 16, 64,
                                    strides3((16 * 2 * 64, 128, 64)), 64,
                                    strides3((16 * 2 * 64, 128, 64)), 0.125, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_EINVAL
    cu = np.array([0, 10, 500], dtype=np.int32)
    st = L.ca_chunk_attn_varlen_fwd(FAKE, FAKE, FAKE, FAKE, cu.ctypes.data, 100, 1, 2, 16, 64,
                                    strides3((16 * 2 * 64, 128, 64)), 64,
                                    strides3((16 * 2 * 64, 128, 64)), 0.125, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_ERANGE
    st = L.ca_chunk_attn_varlen_fwd(FAKE, FAKE, FAKE, FAKE, None, 100, 1, 2, 16, 64,
                                    strides3((16 * 2 * 64, 128, 64)), 60,
                                    strides3((16 * 2 * 64, 128, 64)), 0.125, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_EINVAL


def test_mixed_mode_checks(L):
    bad = np.array([0, 3], dtype=np.int32)
    st = L.ca_chunk_attn_mixed_fwd(FAKE, FAKE, FAKE, 1, 2, 16, 64, 64, S, S, S, bad.ctypes.data,
                                   None, None, 0, None, None, 0, 64, 64, 64, 64, None, None, None,
                                   None, 0, 64, 0.1, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_EINVAL
    blocks = np.array([1, 1], dtype=np.int32)
    st = L.ca_chunk_attn_mixed_fwd(FAKE, FAKE, FAKE, 1, 2, 16, 64, 64, S, S, S, blocks.ctypes.data,
                                   None, None, 0, None, None, 0, 64, 64, 64, 64, None, None, None,
                                   None, 0, 64, 0.1, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_EINVAL        # block heads without a CSR
    # shared lists for one-pass PBSA: both pointers, and query blocks of at most 64
    st = L.ca_chunk_attn_mixed_fwd(FAKE, FAKE, FAKE, 1, 2, 16, 64, 64, S, S, S, blocks.ctypes.data,
                                   FAKE, FAKE, 1, FAKE, None, 0, 64, 64, 64, 64, None, None, None,
                                   None, 0, 64, 0.1, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_EINVAL        # shared indptr without shared indices
    st = L.ca_chunk_attn_mixed_fwd(FAKE, FAKE, FAKE, 1, 2, 16, 64, 64, S, S, S, blocks.ctypes.data,
                                   FAKE, FAKE, 1, FAKE, FAKE, 1, 64, 64, 128, 128, None, None,
                                   None, None, 0, 64, 0.1, FAKE, 0, FAKE, 0, None, 0, None)
    assert st == CA_ERANGE        # q_block above 64 with shared lists


def test_workspace_size_query(L):
    assert L.ca_attn_workspace_bytes(96) == 0
    if not torch.cuda.is_available():
        assert L.ca_attn_workspace_bytes(128) == 0       # no device


def test_merge_mean_topk_index_checks(L):
    s = strides3((1024, 128, 64))
    m = lambda **kw: L.ca_lse_merge(kw.get("o1", FAKE), FAKE, FAKE + 4096, FAKE, kw.get("idt", 1),
                                    kw.get("o", FAKE + 8192), FAKE + 256, kw.get("odt", 0),
                                    1, 2, 8, kw.get("d", 64), s, s, kw.get("os", s), None)
    assert m(d=48) == CA_EUNSUPPORTED
    assert m(idt=3) == CA_EUNSUPPORTED
    assert m(o1=None) == CA_EINVAL
    assert m(o=FAKE + 4096) == CA_EINVAL                      # aliases o2
    assert m(o=FAKE, odt=0) == CA_EINVAL                      # aliases o1 with another dtype
    assert L.ca_block_mean(FAKE, 1, 100, 2, 12, s, 64, 100, FAKE, None, None) == CA_EUNSUPPORTED
    assert L.ca_block_mean(FAKE, 1, 100, 2, 64, s, 0, 100, FAKE, None, None) == CA_EINVAL
    bp = lambda **kw: L.ca_block_mean_pair(FAKE, s, FAKE + 4096, None, kw.get("x2", FAKE + 8192), s,
                                           kw.get("o2", FAKE + 16384), 1, 100, 2, kw.get("d", 64),
                                           64, 100, None)
    assert bp(d=12) == CA_EUNSUPPORTED
    assert bp(x2=None) == CA_EINVAL
    assert bp(o2=None) == CA_EINVAL
    assert bp(x2=FAKE + 8) == CA_EINVAL                 # misaligned
    job = lambda **kw: _lib.TopkJob(FAKE, FAKE, 1, 2, kw.get("nqb", 75), 525, 128, kw.get("cb", 450),
                                    75, kw.get("K", 10), kw.get("pb", 0), kw.get("pc", 0),
                                    kw.get("off", 0), FAKE, None, kw.get("ip", None),
                                    kw.get("ix", None))
    def batch(*jobs):
        arr = (_lib.TopkJob * len(jobs))(*jobs)
        return L.ca_block_score_topk_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), None)
    assert L.ca_block_score_topk_batch(None, 1, None) == CA_EINVAL
    assert batch(*[job()] * 5) == CA_ERANGE             # more than 4 jobs
    assert batch(job(), job(K=0)) == CA_ERANGE          # second job checked too
    assert batch(job(cb=451)) == CA_ERANGE
    assert batch(job(ip=FAKE)) == CA_EINVAL             # lists without indices
    assert batch(job(ip=FAKE, ix=FAKE, pc=451)) == CA_EINVAL   # prefix reaches the candidates
    t = lambda **kw: L.ca_block_score_topk(FAKE, FAKE, 1, 2, 75, 525, 128, kw.get("cb", 450),
                                           kw.get("cc", 75), kw.get("K", 10), FAKE, None, None)
    assert t(K=0) == CA_ERANGE
    assert t(K=76) == CA_ERANGE
    assert t(cb=451) == CA_ERANGE
    assert t(cc=5000) == CA_ERANGE
    assert L.ca_build_kv_index(1, 2, 75, 0, 25, None, 32, FAKE, 10, 0, FAKE, FAKE, None) == CA_EINVAL
    tl = lambda **kw: L.ca_block_score_topk_lists(FAKE, FAKE, 1, 2, 75, 525, 128, kw.get("cb", 25),
                                                  425, 32, kw.get("pb", 0), kw.get("pc", 25),
                                                  kw.get("off", 0), FAKE, kw.get("ip", FAKE),
                                                  FAKE, None)
    assert tl(ip=None) == CA_EINVAL
    assert tl(pc=26) == CA_EINVAL                      # prefix reaches the first candidate id
    assert tl(pc=-1) == CA_EINVAL
    assert tl(off=-26) == CA_ERANGE
    assert tl(pb=10, pc=10, off=-6) == CA_EINVAL       # prefix end 20 > first id -6 + 25
    u = lambda **kw: L.ca_persistent_update(FAKE, FAKE, 1, 12, 525, kw.get("d", 128), kw.get("p", FAKE),
                                            kw.get("cin", 32), kw.get("eb", 450), kw.get("ne", 75),
                                            kw.get("C", 32), kw.get("out", FAKE + 4096), None, None)
    assert u(d=6) == CA_EUNSUPPORTED
    assert u(p=None) == CA_EINVAL                      # C_in > 0 without persistent ids
    assert u(eb=460) == CA_ERANGE                      # evicted range past NKB
    assert u(C=0) == CA_ERANGE
    assert u(out=FAKE, C=16) == CA_EINVAL              # in place with a different C
    assert L.ca_build_kv_index(1, 1000, 75, 0, 25, FAKE, 32, FAKE, 10, 0, FAKE, FAKE, None) == CA_ERANGE


def test_binding_rejects_cpu_tensors():
    import kv_cache_attention_chunk_amd as ca
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ca.chunk_attn_fwd(q, q, q)


def test_header_is_plain_c_and_links(tmp_path):
    """The header compiles as C99 (no C++ in the interface) and a C program
    that calls through it links against the library and runs its host-only
    entry points."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text('#include "chunkattn.h"\n#include <stdio.h>\n'
                   'int main(void) {\n'
                   '  if (ca_abi_version() != CA_ABI_VERSION) return 1;\n'
                   '  if (ca_num_blocks(1560, 64, 1560) != 25) return 2;\n'
                   '  printf("%s\\n", ca_status_str(CA_ERANGE));\n'
                   '  return 0;\n}\n')
    exe = tmp_path / "abi"
    pkg = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I",
                        os.path.join(os.path.dirname(pkg), "include"), str(src), "-L", pkg,
                        "-lchunkattn", f"-Wl,-rpath,{pkg}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip() == "value out of range"

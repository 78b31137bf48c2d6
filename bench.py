#!/usr/bin/env python3
"""Benchmark of the chunk-attention hot path on one MI355X.

Workload: the Wan-1.3B-shaped layer -- 12 heads, d = 128, a 3-frame query
chunk (4680 tokens) against a 21-frame KV cache (32760 tokens), bf16 inputs
N(0,1) with a per-head scale in [0.5, 2] on Q and K, seed 0, resident in HBM.

One step = one pass over every step of the path on that batch:
  1. dense chunk attention -> O (bf16), LSE
  2. local branch (sink + chunk frames) and history branch (frames 1..17) as
     block-list attention with float32 outputs, then the LSE merge -> O, LSE
  3. block-sparse path: block means of Q and of the chunk's own K (the
     history key-block means are resident cache state, built once before the
     timed region), chunk-mean query, top-C persistent history blocks, top-K
     local blocks (K = 12.5 % of 75), block-list assembly, block-list
     attention -> O, LSE

`value` is the step's algorithmic attention FLOPs (4 d per query-key score
over every key set attended) divided by the step time.  The roofline entry
is the dense attention kernel (the dominant kernel), timed with HIP events on
the launch stream over the timed steps, against the datasheet peak and
against the peaks measured here (an MFMA-loop probe, a large GEMM).

After the step, every other workload is timed on its own (warm, and cold
over rotating input copies), and its outputs at sampled query rows are
kept.  The CPU leg then times the float64 oracle on the full dense layer
(the baseline's value), compares every element of the step's dense output
with it, and recomputes each kept sample: max |dO|, max |dLSE|, elements
that needed the relaxed bf16 bound, and for the block-sparse workloads the
top-K rows that differ from the oracle's selection and its near-tie rows.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "kv_cache_attention_chunk_amd", "csrc")
ATTN_SRC = [os.path.join(CSRC, f) for f in ("attn_fwd.hip", "attn_tile.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(paths=None) -> str:
    """Hash of a kernel's code (by default the dense attention kernel:
    attn_fwd.hip and its tile loop attn_tile.h) with // comments, surrounding
    whitespace and blank lines removed, so that counters stay attached to the
    code they were taken on and not to its comments."""
    lines = []
    for path in paths or ATTN_SRC:
        for line in open(path, encoding="utf-8").read().splitlines():
            code = line.split("//", 1)[0].strip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def traffic_from_counters():
    """Bytes per dense call (its attention launch; the plain grid has no
    split merge) from the committed rocprofv3 counter runs, if they were
    taken on the current kernel code; else None."""
    c = counters("attn_fwd_dense_wan", ("attn_fwd.hip", "attn_tile.h"))
    return None if c is None else c.get("hbm_bytes_per_call")


def effective_schedule(ca, q, k, v, scale, policy):
    """Which schedule a dense call under `policy` runs: its output is compared
    bit for bit with the plain grid's and the balanced schedule's (the two
    round split query tiles differently)."""
    import torch
    outs = {}
    for name, pol in (("run", policy), ("plain", "never"), ("balanced", "always")):
        outs[name] = ca.chunk_attn_fwd(q, k, v, scale=scale, balanced=pol)
    torch.cuda.synchronize()
    for name in ("plain", "balanced"):
        if all(torch.equal(a, b) for a, b in zip(outs["run"], outs[name])):
            return name
    return "unknown"


def _cpu_info():
    """The host CPU model, the threads the oracle's numpy BLAS runs with,
    and which BLAS library that is."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads, blas = len(os.sched_getaffinity(0)), "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            threads = max(int(i.get("num_threads", 1)) for i in libs)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
    except Exception:
        pass
    return model, threads, blas


def _o_stats(og, o_ref, bf16_out):
    """max |dO| and, against the O bar (1e-2; for a bf16 output from
    |O_ref| = 2 on 1e-2 plus the output's half-ulp), the elements that
    needed the relaxed bound and those beyond any bound."""
    og = np.asarray(og, np.float64)
    err = np.abs(og - o_ref)
    ax = np.abs(o_ref)
    hu = np.where(ax > 0, 2.0 ** (np.floor(np.log2(np.where(ax > 0, ax, 1.0))) - 8), 0.0)
    bound = np.where(bf16_out & (ax >= 2.0), 1e-2 + hu, 1e-2)
    return {"max_abs_dO": float(np.nanmax(err)) if err.size else 0.0,
            "o_elements": int(err.size),
            "o_relaxed_bound": int(np.sum((err > 1e-2) & (err <= bound))),
            "o_over_bar": int(np.sum(~(err <= bound)))}


def _lse_stats(lg, l_ref):
    """max |dLSE| over finite entries, entries beyond 1e-3, and whether the
    -inf entries (empty key sets) coincide."""
    lg = np.asarray(lg, np.float64)
    fin = np.isfinite(l_ref)
    err = np.abs(lg[fin] - l_ref[fin])
    return {"max_abs_dLSE": float(np.nanmax(err)) if err.size else 0.0,
            "lse_over_bar": int(np.sum(~(err <= 1e-3))),
            "lse_neginf_match": bool(np.array_equal(np.isneginf(lg), np.isneginf(l_ref)))}


def _topk_stats(ig, ref, eps=1e-4):
    """Selected-id rows that differ from the oracle's; those whose differing
    ids are not explained by a near-tie (the K-th/(K+1)-th score gap below
    eps, the set holding every candidate above the tie band and nothing
    below it); and the oracle's near-tie rows."""
    ig = np.asarray(ig)
    diff = np.any(ig != ref["idx"], axis=-1)
    unexplained = 0
    for pos in zip(*np.nonzero(diff)):
        ok = bool(ref["gap"][pos] < eps)
        if ok:
            score_of = {int(c): float(x) for c, x in zip(ref["cand"][pos], ref["cand_score"][pos])
                        if c >= 0}
            kth = float(ref["kth"][pos])
            got = [int(x) for x in ig[pos] if x >= 0]
            must = {c for c, x in score_of.items() if x > kth + eps}
            ok = must <= set(got) and all(c in score_of and score_of[c] >= kth - eps for c in got)
        unexplained += not ok
    return {"rows": int(diff.size), "rows_differing": int(diff.sum()),
            "rows_differing_outside_tie_band": int(unexplained),
            "near_tie_rows": int(np.sum(ref["gap"] < eps))}


def _oracle_for(oracle, spec, rows):
    """The oracle's O and LSE at `rows` for a probe's workload, and what it
    decided on the way (block selections), as the pages define them."""
    kind, extra = spec["kind"], {}
    if kind in ("dense", "merge", "local", "sparse"):
        w = spec["w"]
        Q, K, V = w.q.f32, w.k.f32, w.v.f32
    if kind == "dense":
        O, L = oracle.chunk_attn_dense(Q, K, V, w.scale, rows=rows)
    elif kind in ("merge", "local"):
        spans = oracle.block_spans(w.Nkv, 64, spec.get("seg", 1560))
        br = []
        for key in ("local_blocks", "history_blocks")[:1 if kind == "local" else 2]:
            tok = oracle.block_tokens(spans, w.meta[key])
            br.append(oracle.chunk_attn_dense(Q[:, rows], K[:, tok], V[:, tok], w.scale))
        O, L = br[0] if kind == "local" else oracle.lse_merge_bshd(br[0][0], br[0][1],
                                                                     br[1][0], br[1][1])
    elif kind == "sparse":
        sel = oracle.sparse_selection(Q, K, 64, 1560, 64, 1560, spec["lay"])
        extra["sel"] = sel
        O, L = oracle.chunk_attn_blocks(Q, K, V, sel["indptr"], sel["indices"], 64, 1560, 64,
                                        1560, w.scale, rows=rows)
    elif kind == "varlen":
        w = spec["w"]
        O, L = oracle.chunk_attn_varlen(w.q.f32, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens,
                                        w.scale, rows=rows)
    elif kind == "mixed":
        w, lay, hs = spec["w"], spec["lay"], spec["sparse_heads"]
        Q, K, V = w.q.f32, w.k.f32, w.v.f32
        sel = oracle.sparse_selection(Q[:, :, hs], K[:, :, hs], 64, 1560, 64, 1560, lay)
        extra["sel"] = sel
        O = np.zeros((w.B, len(rows), w.H, w.d))
        L = np.zeros((w.B, w.H, len(rows)))
        for mode in range(3):
            heads = [h for h in range(w.H) if w.head_mode[h] == mode]
            if mode == 0:
                o, l = oracle.chunk_attn_dense(Q, K, V, w.scale, rows=rows, heads=heads)
            elif mode == 1:
                o, l = oracle.chunk_attn_blocks(Q[:, :, hs], K[:, :, hs], V[:, :, hs],
                                                sel["indptr"], sel["indices"], 64, 1560, 64,
                                                1560, w.scale, rows=rows)
            else:
                o, l = oracle.chunk_attn_varlen(Q, w.k_flat.f32, w.v_flat.f32, w.cu_seqlens,
                                                w.scale, rows=rows, heads=heads)
            O[:, :, heads], L[:, heads] = o, l
    else:
        raise ValueError(kind)
    return O, L, extra


def cpu_baseline(w, dense_o=None, dense_l=None, probes=None):
    """The CPU oracle, as it stands, on a bounded sample of the workload,
    timed on this host, and its comparison with the GPU outputs.

    `value`: the full dense Wan layer (12 heads, all 4680 query rows vs 32760
    keys) in float64 numpy, as algorithmic TFLOP/s; with the step's dense
    output (dense_o, dense_l) every one of its elements is compared.  Then,
    per probe the GPU leg stored: the oracle's time, max |dO| and max |dLSE|
    at the sampled rows with the elements that needed the relaxed bf16 bound
    and those beyond any bound, and for the block-sparse workloads the
    top-K rows that differ from the oracle's selection and its near-tie rows
    (ties within 1e-4 of the K-th score)."""
    import oracle
    model, threads, blas = _cpu_info()
    Q, K, V = w.q.f32, w.k.f32, w.v.f32
    oracle.chunk_attn_dense(Q, K, V, w.scale, rows=np.arange(8), heads=[0])    # warm-up
    t0 = time.perf_counter()
    O, L = oracle.chunk_attn_dense(Q, K, V, w.scale)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * w.H * w.Nq * w.Nkv
    per = {}
    if dense_o is not None:
        per["wan_dense_whole_layer"] = {"oracle_ms": round(dt * 1e3, 1), "rows": int(w.Nq),
                                        **_o_stats(dense_o, O, True), **_lse_stats(dense_l, L)}
    del O, L
    t_all = dt
    for name, pr in (probes or {}).items():
        spec = pr["spec"]
        t0 = time.perf_counter()
        rec = {}
        if spec["kind"] == "pack":
            ww = spec["w"]
            frames = [ww.ragged_frames[bh] for bh in range(ww.B * ww.H)]
            ptr = np.zeros(len(frames) + 1, np.int64)
            src = []
            for bh, fl in enumerate(frames):
                for fr in fl:
                    src.append((int(fr[0]), int(fr[1])) if isinstance(fr, (tuple, list))
                               else (int(fr), -1))
                ptr[bh + 1] = len(src)
            rk, rv, rcu = oracle.pack_ragged(ww.k.bits, ww.v.bits, ptr,
                                             np.array(src, np.int64).reshape(-1, 2), 1560)
            rec = {"elements": int(rk.size + rv.size),
                   "elements_differing": int(np.sum(rk != pr["k"]) + np.sum(rv != pr["v"])),
                   "cu_seqlens_equal": bool(np.array_equal(rcu, pr["cu"]))}
        elif spec["kind"] == "persistent":
            ww, lay = spec["w"], spec["lay"]
            qm = oracle.chunk_mean_query(ww.q.f32).astype(np.float32)
            km = oracle.block_mean(ww.k.f32, 64, 1560).astype(np.float32)
            pers = oracle.block_score_topk(qm, km, lay["hist_begin"], lay["hist_count"], lay["C"])
            ref = oracle.persistent_update(qm, km, pers["idx"][:, :, 0, :], lay["local_begin"],
                                           lay["local_count"], lay["C"])
            rec = {"topk": _topk_stats(pr["ids"], ref)}
        elif spec["kind"] == "mla":
            m = spec["m"]
            kv = m["kv_lat"].f32
            o_err, l_err = [], []
            for h, r in spec["rows_by_head"].items():
                Or, Lr = oracle.mla_chunk_attn(m["q"].f32, kv[..., :192], kv[..., 192:],
                                               m["w_uk"].f32, m["w_uv"].f32, m["scale"],
                                               rows=r, heads=[h])
                o_err.append(_o_stats(pr["o"][h], Or, True))
                l_err.append(_lse_stats(pr["lse"][h], Lr))
            rec = {"rows": int(sum(len(r) for r in spec["rows_by_head"].values())),
                   "max_abs_dO": max(x["max_abs_dO"] for x in o_err),
                   "o_elements": sum(x["o_elements"] for x in o_err),
                   "o_relaxed_bound": sum(x["o_relaxed_bound"] for x in o_err),
                   "o_over_bar": sum(x["o_over_bar"] for x in o_err),
                   "max_abs_dLSE": max(x["max_abs_dLSE"] for x in l_err),
                   "lse_over_bar": sum(x["lse_over_bar"] for x in l_err),
                   "lse_neginf_match": all(x["lse_neginf_match"] for x in l_err)}
        else:
            O, L, extra = _oracle_for(oracle, spec, pr["rows"])
            rec = {"rows": int(len(pr["rows"])), **_o_stats(pr["o"], O, pr["bf16_out"]),
                   **_lse_stats(pr["lse"], L)}
            if "sel" in extra:
                sel = extra["sel"]
                rec["topk_persistent"] = _topk_stats(pr["persistent"], sel["persistent"])
                rec["topk_local"] = _topk_stats(pr["local"], sel["local"])
        dt_p = time.perf_counter() - t0
        t_all += dt_p
        per[name] = {"oracle_ms": round(dt_p * 1e3, 1), **rec}
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full dense layer ({w.H} heads x {w.Nq} queries x {w.Nkv} keys), "
                      f"float64 numpy oracle, {dt:.1f} s; then the per-workload parity "
                      f"samples ({t_all - dt:.1f} s)",
            "cpu_model": model, "blas": blas, "oracle_s_total": round(t_all, 1),
            "parity": per}


class _Timing(float):
    """Average time per call in ms, carrying the median and the minimum of
    single-launch timings (None when not taken)."""
    median = None
    minimum = None


def _time_ms(torch, fn, reps=10, warmup_s=0.2, spread=True):
    """Average HIP-event time of fn() on the current stream, in ms, after
    about warmup_s seconds of untimed calls (clocks settle under load); with
    spread, also the median and minimum over 20 calls timed one by one."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warmup_s:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    t = _Timing(e0.elapsed_time(e1) / reps)
    if spread:
        calls = _time_calls(torch, lambda i=0: fn(), 20, 0.0)
        t.median, t.minimum = float(np.median(calls)), float(calls.min())
    return t


def _graphed(torch, fn):
    """fn's launches captured once into a HIP graph (torch.cuda.CUDAGraph),
    after an eager warm-up on a side stream; returns the replay function.
    The library's calls launch kernels only, so they capture as they are."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay


def _time_calls(torch, fn, reps=20, warmup_s=0.2):
    """Per-call HIP-event times of fn() in ms (one event pair per call, on the
    current stream), after about warmup_s seconds of untimed calls."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warmup_s:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(s)
        fn(i)
        ev[i][1].record(s)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def measured_roofs(torch):
    """Roofs measured on this GPU: the bf16 matrix-core peak from an
    MFMA-loop probe (four independent v_mfma_f32_32x32x16_bf16 chains per
    wave, 16 waves per CU, held for about 0.5 s so that the clock settles
    under load), the MFMA rate of the attention tile loop's instruction mix
    with nothing else in the way (its ceiling on this chip), the HBM read
    bandwidth from a streaming-read probe over
    4 GiB, and for reference a large bf16 GEMM (torch.matmul, 8192^3) and a
    1 GiB device-to-device copy."""
    import ctypes
    roofs_lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_attention_chunk_amd",
                                         "libchunkattn_roofs.so"))
    roofs_lib.ca_roof_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    roofs_lib.ca_roof_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    roofs_lib.ca_roof_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(1 << 20, device="cuda", dtype=torch.float32)
    grid, iters = 1024, 20000
    flop = grid * 4 * iters * 4 * 32768.0
    mfma = lambda: roofs_lib.ca_roof_mfma(grid, iters, sink.data_ptr(), stream)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        mfma()
        torch.cuda.synchronize()
    ms_m = _time_ms(torch, mfma, 20, warmup_s=0.0, spread=False)
    grid_x, iters_x = 512, 20000
    flop_x = grid_x * 4 * iters_x * 4 * 32768.0
    mix = lambda: roofs_lib.ca_roof_mix(grid_x, iters_x, sink.data_ptr(), stream)
    ms_x = _time_ms(torch, mix, 20, warmup_s=0.3, spread=False)
    n_read = 4 << 30
    x = torch.empty(n_read // 2, device="cuda", dtype=torch.bfloat16)
    read = lambda: roofs_lib.ca_roof_read(x.data_ptr(), n_read, 8192, sink.data_ptr(), stream)
    ms_r = _time_ms(torch, read, 20, spread=False)
    del x
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    ms_g = _time_ms(torch, lambda: torch.matmul(a, b, out=c), 20, spread=False)
    del a, b, c
    n = 1 << 29                                  # 1 GiB of bf16
    x = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    y = torch.empty_like(x)
    ms_c = _time_ms(torch, lambda: y.copy_(x), 20, spread=False)
    del x, y
    return {"mfma_loop_tflops": round(flop / (ms_m * 1e-3) / 1e12, 1),
            "tile_mix_tflops": round(flop_x / (ms_x * 1e-3) / 1e12, 1),
            "hbm_read_GBs": round(n_read / (ms_r * 1e-3) / 1e9, 1),
            "bf16_gemm_tflops": round(2.0 * 8192 ** 3 / (ms_g * 1e-3) / 1e12, 1),
            "copy_GBs": round(2.0 * (1 << 30) / (ms_c * 1e-3) / 1e9, 1),
            "mfma_loop": "4 chains of v_mfma_f32_32x32x16_bf16 per wave, 1024 x 4 waves, "
                         "after 0.5 s under load",
            "tile_mix": "the attention tile loop's per-MFMA mix (LDS operand reads incl. "
                        "transposing ones, exp2, FMA, add, max, bf16 pack) without memory "
                        "traffic, barriers or dependencies, 2 waves per SIMD",
            "hbm_read": "4 GiB streamed once, 16-byte coalesced loads",
            "gemm": "torch.matmul bf16 8192x8192x8192", "copy": "1 GiB read + 1 GiB written"}


def _sample_rows(Nq, block=None, seg=None, seed=0):
    """Query rows for the parity samples: one random row in every 32-row
    slice of the 256-row query tiles (every wave of every dense / ragged
    workgroup) and, with a query-block tiling, in every 32-row slice of
    every query block (block-list workgroups), plus the first and last."""
    rng = np.random.default_rng(seed)
    rows = {0, Nq - 1}
    for s0 in range(0, Nq, 32):
        rows.add(int(rng.integers(s0, min(s0 + 32, Nq))))
    if block:
        bps = -(-seg // block)
        for j in range(-(-Nq // seg) * bps):
            f, r = divmod(j, bps)
            s0 = f * seg + r * block
            ln = min(block, seg - r * block, Nq - s0)
            for o in range(0, max(ln, 0), 32):
                rows.add(int(rng.integers(s0 + o, s0 + min(o + 32, ln))))
    return np.array(sorted(rows), dtype=np.int64)


def _probe(o, lse, rows, spec, bf16_out=True, **extra):
    """GPU outputs O [B, R, H, d] and LSE [B, H, R] at the sampled rows R,
    kept with the workload description `spec` for the CPU leg's comparison
    (extra: the block ids the GPU selected, as host arrays)."""
    d = {"rows": rows, "o": o[:, rows].float().cpu().numpy(), "lse": lse[:, :, rows].cpu().numpy(),
         "spec": spec, "bf16_out": bf16_out}
    d.update(extra)
    return d


def _time_cold(torch, fn_of_set, n_sets, reps=30):
    """Median and minimum of single calls that rotate over n_sets input
    copies, so that no call finds its K/V in the Infinity Cache or L2."""
    t = _time_calls(torch, lambda i=0: fn_of_set(i % n_sets), reps)
    return round(float(np.median(t)), 4), round(float(t.min()), 4)


def _block_len(ids, block=64, seg=1560):
    """Tokens of frame-aligned block ids (25 blocks per 1560-token frame)."""
    bps = -(-seg // block)
    return np.minimum(block, seg - block * (np.asarray(ids) % bps))


def _rec(ms, flops, kv_bytes, **extra):
    r = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
         "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
         "kv_GBs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
         "kv_frac_hbm": round(kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
         "gflop": round(flops / 1e9, 2), "kv_MB": round(kv_bytes / 1e6, 2)}
    if getattr(ms, "median", None) is not None:
        r["ms_median"] = round(ms.median, 4)
        r["ms_min"] = round(ms.minimum, 4)
    r.update(extra)
    return r


def _cold_sets(touched_bytes):
    """Input copies a cold timing rotates over: enough that the other copies'
    K/V bytes read between two uses of one copy exceed twice the 256 MB
    Infinity Cache (at least 3 copies, at most 12)."""
    return int(min(12, max(3, 1 + math.ceil(2 * 256e6 / max(touched_bytes, 1.0)))))


def _add_cold(torch, rec, flops, call, n_sets, reps=30):
    """Cold timing of call(i) (i = the input copy) added to a record."""
    med, mn = _time_cold(torch, call, n_sets, reps)
    rec.update(cold_ms_median=med, cold_ms_min=mn, cold_sets=n_sets,
               cold_tflops_median=round(flops / (med * 1e-3) / 1e12, 1))


def counters(name, sources):
    """A workload's committed rocprofv3 counter summary
    (profiles/<name>_counters.json) if it was taken on the current code of
    `sources` (paths under csrc/); else None."""
    try:
        c = json.load(open(os.path.join(ROOT, "profiles", f"{name}_counters.json")))
    except (OSError, ValueError):
        return None
    if c.get("code_sha256_16") != src_hash([os.path.join(CSRC, s) for s in sources]):
        return None
    return c


SPARSE_SOURCES = ("pbsa.hip", "attn_tile.h", "select.hip", "common.h")


def per_config(reps=10, wan=None, names=None, probes=None):
    """Time every configured workload on the GPU (inputs resident): tiny dense
    + merge, Wan dense / merge / dual output, block-sparse at three top-K
    ratios, persistent update, ragged, ragged packing, latent-KV (MLA),
    mixed 40-head.  FLOPs are algorithmic (4 d per score of every key set
    attended); kv bytes are the distinct K/V bytes the call must read.
    Attention workloads also get a cold timing over rotating input copies
    (no K/V left in the Infinity Cache or L2 from the call before).

    With `probes` (a dict), each workload's outputs at sampled query rows
    (every wave slice of every workgroup), its selected block ids and what
    an oracle needs to recompute them are stored there, for the CPU leg to
    compare.  `names` restricts the run to those entries (for per-workload
    counter collection); their inputs are still built."""
    import torch
    import kv_cache_attention_chunk_amd as ca
    from kv_cache_attention_chunk_amd import workloads as wl
    want = lambda n: names is None or n in names
    dev = lambda t: torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    probes = {} if probes is None else probes
    out = {}

    def merged_fn(q, k, v, w, seg, om, lm):
        br = []
        for key in ("local_blocks", "history_blocks"):
            blocks = np.array(w.meta[key], np.int32)
            BH = w.B * w.H
            br.append((i32(np.arange(BH + 1) * len(blocks)), i32(np.tile(blocks, BH)),
                       f32(w.B, w.Nq, w.H, w.d), f32(w.B, w.H, w.Nq)))

        def fn():
            for ip, ix, ob, lb in br:
                ca.chunk_attn_fwd(q, k, v, kv_indptr=ip, kv_indices=ix, kv_block=64, kv_seg=seg,
                                  q_block=w.Nq, q_seg=w.Nq, scale=w.scale,
                                  out_dtype=torch.float32, out=ob, lse=lb)
            ca.lse_merge(br[0][2], br[0][3], br[1][2], br[1][3], out=om, out_lse=lm)
        return fn

    # tiny dense chunk (launch-latency scale; no roofline claim)
    w = wl.tiny_dense(seed=0)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    f = 4.0 * w.d * w.Nq * w.Nkv * w.B * w.H
    if want("tiny_dense"):
        od, ld = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        om, lm = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        dense_fn = lambda: ca.chunk_attn_fwd(q, k, v, scale=w.scale, out=od, lse=ld)
        merge_fn = merged_fn(q, k, v, w, w.Nkv, om, lm)
        ms_d = _time_ms(torch, dense_fn, reps)
        ms_m = _time_ms(torch, merge_fn, reps)
        # the same calls replayed from a HIP graph: the launch-latency scale
        # without the per-call host work (argument checks, ctypes, launch)
        ms_dg = _time_ms(torch, _graphed(torch, dense_fn), reps)
        ms_mg = _time_ms(torch, _graphed(torch, merge_fn), reps)
        out["tiny_dense"] = {"dense_us": round(ms_d * 1e3, 1),
                             "local_history_merge_us": round(ms_m * 1e3, 1),
                             "dense_graph_us": round(ms_dg * 1e3, 1),
                             "local_history_merge_graph_us": round(ms_mg * 1e3, 1),
                             "gflop": round(f / 1e9, 3)}
        rows = np.arange(w.Nq)
        probes["tiny_dense"] = _probe(od, ld, rows, {"kind": "dense", "w": w})
        probes["tiny_merge"] = _probe(om, lm, rows, {"kind": "merge", "w": w, "seg": w.Nkv})

    # Wan-1.3B layer: dense, local/history merge, dual output
    w = wan or wl.wan_dense(seed=0)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    f_dense = 4.0 * w.d * w.Nq * w.Nkv * w.B * w.H
    kvb = 2.0 * w.Nkv * w.H * w.d * 2
    rows = _sample_rows(w.Nq, 64, 1560, seed=1)
    ms_dense = None
    if want("wan_dense"):
        o_w, l_w = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        rec = _rec(_time_ms(torch, lambda: ca.chunk_attn_fwd(q, k, v, scale=w.scale, out=o_w,
                                                             lse=l_w), reps), f_dense, kvb)
        n = _cold_sets(kvb)
        sets = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n - 1)]
        _add_cold(torch, rec, f_dense, lambda i=0: ca.chunk_attn_fwd(
            q, sets[i][0], sets[i][1], scale=w.scale, out=o_w, lse=l_w), n)
        del sets
        out["wan_dense"] = rec
        ms_dense = rec["ms"]
    if want("wan_merge_variant"):
        om, lm = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        out["wan_merge_variant"] = _rec(_time_ms(torch, merged_fn(q, k, v, w, 1560, om, lm), reps),
                                        f_dense, kvb)
        probes["wan_merge_variant"] = _probe(om, lm, rows, {"kind": "merge", "w": w, "seg": 1560})
    # local (sink + chunk frames) and full attention from one pass over each head's list
    row = np.array(w.meta["local_blocks"] + w.meta["history_blocks"], np.int32)
    dip, dix = i32(np.arange(w.B * w.H + 1) * len(row)), i32(np.tile(row, w.B * w.H))
    n_loc = len(w.meta["local_blocks"])
    f_loc = 4.0 * w.d * w.Nq * w.B * w.H * float(_block_len(w.meta["local_blocks"]).sum())
    if want("wan_dual_output"):
        ol, ll = f32(w.B, w.Nq, w.H, w.d), f32(w.B, w.H, w.Nq)
        of, lf = f32(w.B, w.Nq, w.H, w.d), f32(w.B, w.H, w.Nq)
        out["wan_dual_output"] = _rec(_time_ms(torch, lambda: ca.chunk_attn_dual_fwd(
            q, k, v, dip, dix, n_loc, kv_block=64, kv_seg=1560, q_block=w.Nq, q_seg=w.Nq,
            scale=w.scale, out_local=ol, lse_local=ll, out=of, lse=lf), reps), f_dense, kvb,
            local_gflop_shared=round(f_loc / 1e9, 2))
        probes["wan_dual_full"] = _probe(of, lf, rows, {"kind": "dense", "w": w}, bf16_out=False)
        probes["wan_dual_local"] = _probe(ol, ll, rows, {"kind": "local", "w": w},
                                          bf16_out=False)

    # block-sparse path at the three top-K ratios (selection included)
    km = ca.block_mean(k, 64, 1560)
    nqb = ca.num_blocks(w.Nq, 64, 1560)
    qlen = np.tile(_block_len(np.arange(nqb)), w.B * w.H)
    cnt = counters("block_sparse_wan", SPARSE_SOURCES)
    for ratio in (0.25, 0.125, 0.0625):
        lay = wl.sparse_layout(w, ratio)
        name = f"sparse_K{lay['K']}"
        if not want(name):
            continue
        o_s, l_s = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        args = dict(sink_begin=0, sink_count=lay["sink_count"], hist_begin=lay["hist_begin"],
                    hist_count=lay["hist_count"], C=lay["C"], local_begin=lay["local_begin"],
                    local_count=lay["local_count"], K=lay["K"], block=64, seg=1560, k_mean=km,
                    scale=w.scale)
        ws = torch.empty(ca.block_sparse_workspace(w.B, w.H, w.Nq, w.Nkv, w.d, block=64,
                                                   seg=1560, have_k_mean=True,
                                                   **{a: args[a] for a in (
                                                       "sink_begin", "sink_count", "hist_begin",
                                                       "hist_count", "C", "local_begin",
                                                       "local_count", "K")}).bytes,
                         dtype=torch.uint8, device="cuda")
        fn = lambda kk=k, vv=v: ca.block_sparse_fwd(q, kk, vv, out=o_s, lse=l_s, workspace=ws,
                                                    **args)
        _, _, info = fn()
        torch.cuda.synchronize()
        sp, sx = info["shared_indptr"].cpu().numpy(), info["shared_indices"].cpu().numpy()
        lp, lx = info["local_indptr"].cpu().numpy(), info["local_indices"].cpu().numpy()
        sh = np.array([_block_len(sx[sp[r]:sp[r + 1]]).sum() for r in range(w.B * w.H)])
        lo = np.array([_block_len(lx[lp[r]:lp[r + 1]]).sum() for r in range(w.B * w.H * nqb)])
        f = 4.0 * w.d * (float(sh.sum()) * w.Nq + float((lo * qlen).sum()))
        uniq = sum(_block_len(np.union1d(sx[sp[h]:sp[h + 1]], lx[lp[h * nqb]:lp[(h + 1) * nqb]])).sum()
                   for h in range(w.B * w.H))
        kvb_s = 2.0 * float(uniq) * w.d * 2
        # bytes the PBSA kernel streams from L2 into LDS: each workgroup (four
        # query blocks of a head) reads its head's shared list once, and each
        # query block its own local list
        groups = -(-nqb // 4)
        gathered = 2.0 * w.d * 2 * (groups * float(sh.sum()) + float(lo.sum()))
        ms = _time_ms(torch, fn, reps)
        # PBSA alone, on the lists the path built
        o_p, l_p = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        lists = [info[x].clone() for x in ("shared_indptr", "shared_indices", "local_indptr",
                                          "local_indices")]
        ms_p = _time_ms(torch, lambda: ca.chunk_attn_pbsa_fwd(
            q, k, v, *lists, kv_block=64, kv_seg=1560, q_block=64, q_seg=1560, scale=w.scale,
            out=o_p, lse=l_p), reps)
        rec = _rec(ms, f, kvb_s, ratio=ratio, K=lay["K"], C=lay["C"],
                   pbsa_ms=round(ms_p, 4), selection_ms=round(ms - ms_p, 4),
                   pbsa_tflops=round(f / (ms_p * 1e-3) / 1e12, 1),
                   gathered_MB=round(gathered / 1e6, 2),
                   gathered_GBs_pbsa=round(gathered / (ms_p * 1e-3) / 1e9, 1))
        if ms_dense is not None:
            rec["speedup_vs_dense"] = round(ms_dense / ms, 2)
        n = _cold_sets(kvb_s)
        sets = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n - 1)]
        _add_cold(torch, rec, f, lambda i=0: fn(*sets[i]), n)
        del sets
        if cnt is not None and name in cnt.get("per_workload", {}):
            c = cnt["per_workload"][name]
            rec["rocprof"] = {"l2_fill_read_MB": c["read_MB"], "write_MB": c["write_MB"],
                              "pbsa_read_MB": c["pbsa_read_MB"],
                              "pbsa_read_over_gathered": round(c["pbsa_read_MB"] * 1e6 / gathered, 3)}
        out[name] = rec
        probes[name] = _probe(o_s, l_s, rows, {"kind": "sparse", "w": w, "lay": lay},
                              persistent=info["persistent"].cpu().numpy(),
                              local=(info["local"] + info["local_base"]).cpu().numpy())
        del ws, o_p, l_p, lists
    # persistent-memory update when the window slides: the chunk's 75 local
    # blocks are evicted into the candidates of each head's 32 persistent blocks
    lay = wl.sparse_layout(w, 0.125)
    _, cm = ca.block_mean(q, 64, 1560, with_total=True)
    pers = ca.block_score_topk(cm, km, lay["C"], cand_begin=lay["hist_begin"],
                               cand_count=lay["hist_count"])[:, :, 0, :].contiguous()
    if want("persistent_update"):
        pn = torch.empty_like(pers)
        ms = _time_ms(torch, lambda: ca.persistent_update(cm, km, pers, lay["local_begin"],
                                                          lay["local_count"], lay["C"], out=pn),
                      reps)
        out["persistent_update"] = {"us": round(ms * 1e3, 1), "us_median": round(ms.median * 1e3, 1),
                                    "us_min": round(ms.minimum * 1e3, 1), "candidates_per_head":
                                    lay["C"] + lay["local_count"], "C": lay["C"], "heads": w.H}
        probes["persistent_update"] = {"spec": {"kind": "persistent", "w": w, "lay": lay},
                                       "ids": pn.cpu().numpy()}
    del q, k, v, km
    # ragged per-head caches
    w = wl.ragged(seed=0)
    q, kf, vf, cu = dev(w.q), dev(w.k_flat), dev(w.v_flat), i32(w.cu_seqlens)
    tot = int(w.cu_seqlens[-1])
    f = 4.0 * w.d * w.Nq * tot
    kvb = 2.0 * tot * w.d * 2
    if want("ragged"):
        o_r, l_r = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        call = lambda i=0, kk=kf, vv=vf: ca.chunk_attn_varlen_fwd(
            q, kk, vv, cu, cu_seqlens_host=w.cu_seqlens, scale=w.scale, out=o_r, lse=l_r)
        rec = _rec(_time_ms(torch, call, reps), f, kvb, sum_len=tot,
                   lengths_frames=w.meta["n_frames"])
        n = _cold_sets(kvb)
        sets = [(kf, vf)] + [(kf.clone(), vf.clone()) for _ in range(n - 1)]
        _add_cold(torch, rec, f, lambda i=0: call(0, *sets[i]), n)
        del sets
        out["ragged"] = rec
        probes["ragged"] = _probe(o_r, l_r, _sample_rows(w.Nq, seed=3), {"kind": "varlen", "w": w})
    # packing those ragged caches from the dense per-head cache (HBM-bound:
    # every packed K/V row read once and written once)
    kd, vd = dev(w.k), dev(w.v)
    plan = ca.pack_plan([w.ragged_frames[bh] for bh in range(w.B * w.H)], kd.device)
    if want("ragged_pack"):
        pk, pv = torch.empty_like(kf), torch.empty_like(vf)
        pcu = torch.empty_like(cu)
        ms = _time_ms(torch, lambda: ca.pack_ragged(kd, vd, plan, 1560, out_k=pk, out_v=pv,
                                                    out_cu=pcu), reps)
        moved = 2.0 * 2.0 * tot * w.d * 2
        out["ragged_pack"] = {"us": round(ms * 1e3, 1), "us_median": round(ms.median * 1e3, 1),
                              "us_min": round(ms.minimum * 1e3, 1), "bytes_moved_MB": round(moved / 1e6, 1),
                              "GBs": round(moved / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        probes["ragged_pack"] = {"spec": {"kind": "pack", "w": w},
                                 "k": pk.view(torch.int16).cpu().numpy().view(np.uint16),
                                 "v": pv.view(torch.int16).cpu().numpy().view(np.uint16),
                                 "cu": pcu.cpu().numpy()}
    del q, kf, vf, kd, vd
    # latent KV cache (d_c = 192, d_rope = 32): absorbed query, latent
    # attention, per-head up-projection
    m = wl.wan_mla(seed=0)
    mq, mwk, mwv = dev(m["q"]), dev(m["w_uk"]), dev(m["w_uv"])
    mkv = ca.cast_bf16_to_f16(dev(m["kv_lat"]))
    if want("wan_mla"):
        o_m, l_m = torch.empty_like(mq), f32(1, m["H"], m["Nq"])
        o_lat = f32(1, m["Nq"], m["H"], 192)
        ms_all = _time_ms(torch, lambda: ca.mla_chunk_attn(mq, mkv, mwk, mwv, scale=m["scale"],
                                                           out=o_m, lse=l_m, o_lat=o_lat), reps)
        rows_m = m["Nq"] * m["H"]
        f_att = 2.0 * rows_m * m["Nkv"] * (224 + 192)
        f_proj = 2.0 * rows_m * (96 * 192 + 192 * 128)
        kvb = m["Nkv"] * 224 * 2.0
        out["wan_mla"] = _rec(ms_all, f_att + f_proj, kvb, attention_gflop=round(f_att / 1e9, 1),
                              projection_gflop=round(f_proj / 1e9, 1),
                              kv_bytes_vs_dense=round(kvb / (2.0 * m["Nkv"] * m["H"] * 128 * 2), 4))
        # one (query, head) row of every 32-row wave slice of the flattened
        # (query, head) rows the latent kernel tiles
        rng = np.random.default_rng(6)
        flat = [int(rng.integers(s, min(s + 32, rows_m))) for s in range(0, rows_m, 32)]
        by_head = {}
        for r in flat:
            by_head.setdefault(r % m["H"], set()).add(r // m["H"])
        og, lg = o_m.float().cpu().numpy(), l_m.cpu().numpy()
        sel = {h: np.array(sorted(rs)) for h, rs in by_head.items()}
        probes["wan_mla"] = {"spec": {"kind": "mla", "m": m, "rows_by_head": sel},
                             "o": {h: og[:, r, h:h + 1] for h, r in sel.items()},
                             "lse": {h: lg[:, h:h + 1, r] for h, r in sel.items()},
                             "bf16_out": True}
    del mq, mwk, mwv, mkv
    # mixed 40-head layer (dense / block lists / ragged per head); the
    # block-sparse heads' lists come from the selection calls on those heads
    w = wl.mixed(seed=0)
    lay = w.meta["sparse"]
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    hs = [h for h in range(w.H) if w.head_mode[h] == 1]
    hsel = torch.tensor(hs, device="cuda")
    qs, ks = q.index_select(2, hsel).contiguous(), k.index_select(2, hsel).contiguous()
    qm, kms, cm = ca.block_mean(qs, 64, 1560), ca.block_mean(ks, 64, 1560), ca.block_mean(qs, w.Nq, w.Nq)
    pers = ca.block_score_topk(cm, kms, lay["C"], cand_begin=lay["hist_begin"], cand_count=lay["hist_count"])
    loc = ca.block_score_topk(qm, kms, lay["K"], cand_begin=lay["local_begin"], cand_count=lay["local_count"])
    ip_s, ix_s = ca.build_kv_index(1, len(hs), nqb, 0, lay["sink_count"], pers[:, :, 0, :].contiguous(), loc, 0)
    ip_s, ix_s = ip_s.cpu().numpy(), ix_s.cpu().numpy()
    sel_gpu = {"persistent": pers.cpu().numpy(), "local": loc.cpu().numpy()}
    del qs, ks
    lists, f, kvb = [], 0.0, 0.0
    for h in range(w.H):
        for qb in range(nqb):
            if w.head_mode[h] == 1:
                r = hs.index(h) * nqb + qb
                lists.append(ix_s[ip_s[r]:ip_s[r + 1]])
            else:
                lists.append(np.zeros(0, np.int32))
        if w.head_mode[h] == 0:
            f += 4.0 * w.d * w.Nq * w.Nkv
            kvb += 2.0 * w.Nkv * w.d * 2
        elif w.head_mode[h] == 1:
            rl = lists[h * nqb:(h + 1) * nqb]
            f += 4.0 * w.d * float(sum(_block_len(x).sum() * ql for x, ql in zip(rl, qlen[:nqb])))
            kvb += 2.0 * float(_block_len(np.unique(np.concatenate(rl))).sum()) * w.d * 2
        else:
            L = int(w.cu_seqlens[h + 1] - w.cu_seqlens[h])
            f += 4.0 * w.d * w.Nq * L
            kvb += 2.0 * L * w.d * 2
    # the block-sparse heads run one-pass PBSA: per head the sink and
    # persistent blocks (shared by its query blocks), per query block its
    # top-K window blocks; the union of the two is the key set of `lists`
    pn, ln = sel_gpu["persistent"], sel_gpu["local"]
    sink = np.arange(lay["sink_count"], dtype=np.int32)
    shared, local = [], []
    for h in range(w.H):
        si = hs.index(h) if w.head_mode[h] == 1 else -1
        shared.append(np.concatenate([sink, pn[0, si, 0]]) if si >= 0 else np.zeros(0, np.int32))
        for qb in range(nqb):
            local.append(ln[0, si, qb] if si >= 0 else np.zeros(0, np.int32))
    csr = lambda rows: (i32(np.concatenate([[0], np.cumsum([len(x) for x in rows])])),
                        i32(np.concatenate(rows)))
    sp, sx = csr(shared)
    lp, lx = csr(local)
    kf, vf, cu = dev(w.k_flat), dev(w.v_flat), i32(w.cu_seqlens)
    if want("mixed_40h"):
        o_x, l_x = torch.empty_like(q), f32(w.B, w.H, w.Nq)
        call = lambda i=0, kk=k, vv=v, kkf=kf, vvf=vf: ca.chunk_attn_mixed_fwd(
            q, w.head_mode, k=kk, v=vv, kv_indptr=lp, kv_indices=lx, kv_shared_indptr=sp,
            kv_shared_indices=sx, kv_block=64, kv_seg=1560, q_block=64, q_seg=1560, k_flat=kkf,
            v_flat=vvf, cu_seqlens=cu, cu_seqlens_host=w.cu_seqlens, scale=w.scale, out=o_x,
            lse=l_x)
        rec = _rec(_time_ms(torch, call, reps), f, kvb,
                   heads_dense_sparse_ragged=[int((w.head_mode == mm).sum()) for mm in range(3)])
        n = _cold_sets(kvb)
        sets = [(k, v, kf, vf)] + [(k.clone(), v.clone(), kf.clone(), vf.clone())
                                   for _ in range(n - 1)]
        _add_cold(torch, rec, f, lambda i=0: call(0, *sets[i]), n)
        del sets
        out["mixed_40h"] = rec
        probes["mixed_40h"] = _probe(o_x, l_x, _sample_rows(w.Nq, 64, 1560, seed=4),
                                     {"kind": "mixed", "w": w, "lay": lay, "sparse_heads": hs},
                                     **sel_gpu)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--topk-ratio", type=float, default=0.125)
    ap.add_argument("--only", choices=["step", "dense", "copy", "configs", "roofs"],
                    default="step",
                    help="'dense' times the dense kernel alone (for counter runs); 'copy' "
                         "runs a plain 1 GiB device copy, the reference for HBM byte counters; "
                         "'roofs' runs the roof probes alone and prints what they measure")
    ap.add_argument("--config", default="",
                    help="with --only configs: comma-separated entries to time (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", choices=["auto", "plain", "balanced"], default="auto",
                    help="dense launch: the library's own choice (default), one workgroup per "
                         "(head, query tile), or the key-range split over the resident "
                         "workgroups")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="with --only dense: keep launching for this many seconds before the "
                         "timed steps (for power and clock sampling)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload timings (tiny, Wan dense/merge, sparse at three "
                         "top-K ratios, ragged, mixed 40-head)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kv_cache_attention_chunk_amd as ca
    from kv_cache_attention_chunk_amd import workloads as wl
    from kv_cache_attention_chunk_amd import _lib
    _lib.lib()

    torch.cuda.set_device(0)
    if args.only == "copy":
        n_bytes = 1 << 30
        x = torch.ones(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            y.copy_(x)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes,
                          "ms": ms, "GBps_read+write": 2 * n_bytes / (ms * 1e-3) / 1e9}))
        return
    if args.only == "roofs":
        print(json.dumps(measured_roofs(torch)), flush=True)
        return
    if args.only == "configs":
        names = set(args.config.split(",")) if args.config else None
        print(json.dumps(per_config(names=names)), flush=True)
        return
    t0 = time.perf_counter()
    w = wl.wan_dense(seed=0)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    dev = lambda t: torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    B, H, Nq, Nkv, d = w.B, w.H, w.Nq, w.Nkv, w.d
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    o_dense = torch.empty_like(q)
    l_dense = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    branch = []
    for key in ("local_blocks", "history_blocks"):
        blocks = np.array(w.meta[key], np.int32)
        branch.append((i32(np.arange(B * H + 1) * len(blocks)), i32(np.tile(blocks, B * H)),
                       torch.empty((B, Nq, H, d), dtype=torch.float32, device="cuda"),
                       torch.empty((B, H, Nq), dtype=torch.float32, device="cuda"), len(blocks)))
    o_merge = torch.empty_like(q)
    l_merge = torch.empty_like(l_dense)
    lay = wl.sparse_layout(w, args.topk_ratio)

    policy = {"auto": "auto", "plain": "never", "balanced": "always"}[args.schedule]

    def dense():
        ca.chunk_attn_fwd(q, k, v, scale=w.scale, out=o_dense, lse=l_dense, balanced=policy)

    def merged():
        for ip, ix, ob, lb, _ in branch:
            ca.chunk_attn_fwd(q, k, v, kv_indptr=ip, kv_indices=ix, kv_block=64, kv_seg=1560,
                              q_block=Nq, q_seg=Nq, scale=w.scale, out_dtype=torch.float32,
                              out=ob, lse=lb)
        ca.lse_merge(branch[0][2], branch[0][3], branch[1][2], branch[1][3], out=o_merge,
                     out_lse=l_merge)

    k_mean_resident = ca.block_mean(k, 64, 1560)

    sparse_ranges = {key: lay[key] for key in ("sink_begin", "sink_count", "hist_begin",
                                               "hist_count", "C", "local_begin", "local_count",
                                               "K")}
    sparse_ws = torch.empty(ca.block_sparse_workspace(B, H, Nq, Nkv, d, block=64, seg=1560,
                                                      have_k_mean=True, **sparse_ranges).bytes,
                            dtype=torch.uint8, device="cuda")
    o_sparse = torch.empty_like(q)
    l_sparse = torch.empty_like(l_dense)

    def sparse():
        return ca.block_sparse_fwd(q, k, v, block=64, seg=1560, k_mean=k_mean_resident,
                                   scale=w.scale, out=o_sparse, lse=l_sparse,
                                   workspace=sparse_ws, **sparse_ranges)

    # algorithmic FLOPs: 4 d per (query, key) score of every key set attended
    f_dense = 4.0 * d * Nq * Nkv * B * H
    f_merge = 4.0 * d * Nq * B * H * sum(
        int(np.minimum(64, 1560 - 64 * (np.array(w.meta[key]) % 25)).sum())
        for key in ("local_blocks", "history_blocks"))
    _, _, info = sparse()
    torch.cuda.synchronize()

    def block_len(j):           # frame-aligned tiling: 25 blocks per 1560-token frame
        r = j % 25
        return np.minimum(64, 1560 - 64 * r)
    nqb = ca.num_blocks(Nq, 64, 1560)
    sp, sx = info["shared_indptr"].cpu().numpy(), info["shared_indices"].cpu().numpy()
    lp, lx = info["local_indptr"].cpu().numpy(), info["local_indices"].cpu().numpy()
    shared_toks = np.array([block_len(sx[sp[r]:sp[r + 1]]).sum() for r in range(B * H)])
    local_toks = np.array([block_len(lx[lp[r]:lp[r + 1]]).sum() for r in range(B * H * nqb)])
    qlen = np.tile(block_len(np.arange(nqb)), B * H)
    f_sparse = 4.0 * d * (float(shared_toks.sum()) * Nq + float((local_toks * qlen).sum()))
    f_step = f_dense + f_merge + f_sparse if args.only == "step" else f_dense

    # which schedule the dense call runs (found before the warm-up, so that a
    # kernel trace of this command averages over the timed launches); the
    # dense-only mode used for counter runs launches nothing else
    schedule = (effective_schedule(ca, q, k, v, w.scale, policy) if args.only == "step"
                else args.schedule)
    stream = torch.cuda.current_stream()
    if args.sustain > 0:
        t_s = time.perf_counter()
        n_s = 0
        while time.perf_counter() - t_s < args.sustain:
            for _ in range(20):
                dense()
            torch.cuda.synchronize()
            n_s += 20
        log(f"sustained {n_s} dense launches over {time.perf_counter() - t_s:.1f} s")
    for _ in range(args.warmup):
        dense()
        if args.only == "step":
            merged()
            sparse()
    torch.cuda.synchronize()

    n = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(n):
        ev[i][0].record(stream)
        dense()
        ev[i][1].record(stream)
        if args.only == "step":
            merged()
            ev[i][2].record(stream)
            sparse()
            ev[i][3].record(stream)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    total_ms = g0.elapsed_time(g1)
    ms_step = total_ms / n
    t_dense = sum(e[0].elapsed_time(e[1]) for e in ev) / n
    res = {"dense_ms": t_dense}
    if args.only == "step":
        res["merge_variant_ms"] = sum(e[1].elapsed_time(e[2]) for e in ev) / n
        res["sparse_path_ms"] = sum(e[2].elapsed_time(e[3]) for e in ev) / n
    log(f"timed {n} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / n:.3f}), {res}")

    # the step's dense output, all of it, for the CPU leg's comparison
    dense_host = (o_dense.float().cpu().numpy(), l_dense.cpu().numpy())
    probes = {}
    achieved = f_dense / (t_dense * 1e-3) / 1e12
    kv_bytes = 2.0 * Nkv * H * d * 2 * B
    traffic = traffic_from_counters()
    out = {
        "metric": "attn TFLOP/s + KV GB/s (% roofline), 4680q×32760kv chunk, 12 heads d128",
        "value": round(f_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan1.3b-shaped chunk attention layer: H=12, d=128, "
                               "Nq=4680 (3 frames), Nkv=32760 (21 frames), bf16 N(0,1), "
                               "per-head Q/K scale U[0.5,2], seed 0",
                   "global_batch": B, "seq_len": Nkv, "parallelism": "none",
                   "step": ("dense + local/history merge + block-sparse(K=%d, C=%d)"
                            % (lay["K"], lay["C"])) if args.only == "step" else "dense only",
                   "step_gflop": round(f_step / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": ("attn_fwd_kernel<128,8,range,bf16> + split_merge_kernel<128,bf16>"
                                if schedule == "balanced" else
                                "attn_fwd_kernel<128,8,range,bf16>"),
                     "schedule": schedule if args.schedule == "auto" else args.schedule,
                     "avg_launch_ms": round(t_dense, 4)},
        "kv_gbs": {"dense": round(kv_bytes / (t_dense * 1e-3) / 1e9, 1),
                   "frac_hbm": round(kv_bytes / (t_dense * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "breakdown_ms": {k_: round(v_, 4) for k_, v_ in res.items()},
        "phase_tflops": {"dense": round(achieved, 1)},
    }
    if args.only == "step":
        out["phase_tflops"]["merge_variant"] = round(f_merge / (res["merge_variant_ms"] * 1e-3) / 1e12, 1)
        out["phase_tflops"]["sparse_path"] = round(f_sparse / (res["sparse_path_ms"] * 1e-3) / 1e12, 1)
    if args.only == "step" and not args.no_configs:
        t0 = time.perf_counter()
        out["configs"] = per_config(wan=w, probes=probes)
        roofs = measured_roofs(torch)
        out["measured_roofs"] = roofs
        out["roofline"]["frac_of_measured_mfma"] = round(achieved / roofs["mfma_loop_tflops"], 4)
        out["roofline"]["frac_of_tile_mix"] = round(achieved / roofs["tile_mix_tflops"], 4)
        out["roofline"]["frac_of_measured_gemm"] = round(achieved / roofs["bf16_gemm_tflops"], 4)
        log(f"per-workload timings in {time.perf_counter() - t0:.1f} s")
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w, dense_host[0], dense_host[1], probes)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f} s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

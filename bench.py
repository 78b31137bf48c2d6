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
the launch stream over the timed steps.  Prints one JSON line.
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
ATTN_SRC = os.path.join(ROOT, "kv_cache_attention_chunk_amd", "csrc", "attn_fwd.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_dense_wan_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash() -> str:
    """Hash of the attention kernel's code: attn_fwd.hip with // comments,
    surrounding whitespace and blank lines removed, so that counters stay
    attached to the code they were taken on and not to its comments."""
    lines = []
    for line in open(ATTN_SRC, encoding="utf-8").read().splitlines():
        code = line.split("//", 1)[0].strip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def traffic_from_counters():
    """HBM bytes per dense call (its attention launch plus the split merge of
    the balanced schedule) from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("attn_fwd_code_sha256_16") != src_hash():
        return None
    return c.get("hbm_bytes_per_call")


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


def cpu_baseline(w):
    """Time the CPU oracle, as it stands, on a bounded sample of the same
    workload: the full dense layer (all 12 heads, all 4680 query rows vs
    32760 keys) plus the oracle's local and history branches and their LSE
    merge over the first 1560 query rows (one latent frame).  Returns the
    baseline record with the achieved algorithmic TFLOP/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    Q, K, V = w.q.f32, w.k.f32, w.v.f32
    oracle.chunk_attn_dense(Q, K, V, w.scale, rows=np.arange(8), heads=[0])    # warm-up
    t0 = time.perf_counter()
    oracle.chunk_attn_dense(Q, K, V, w.scale)
    rows = np.arange(1560)
    tok = {key: oracle.block_tokens(oracle.block_spans(w.Nkv, 64, 1560), w.meta[key])
           for key in ("local_blocks", "history_blocks")}
    br = [oracle.chunk_attn_dense(Q[:, rows], K[:, tok[key]], V[:, tok[key]], w.scale)
          for key in ("local_blocks", "history_blocks")]
    oracle.lse_merge_bshd(br[0][0], br[0][1], br[1][0], br[1][1])
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * w.H * (w.Nq + len(rows)) * w.Nkv
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full dense layer ({w.H} heads x {w.Nq} queries x {w.Nkv} keys) + "
                      f"local/history branches and LSE merge for the first {len(rows)} queries, "
                      f"float64 numpy oracle, {dt:.1f} s"}


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
    """Roofs measured on this GPU: a large bf16 GEMM (torch.matmul, 8192^3,
    contiguous operands) and a 1 GiB device-to-device copy."""
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
    return {"bf16_gemm_tflops": round(2.0 * 8192 ** 3 / (ms_g * 1e-3) / 1e12, 1),
            "copy_GBs": round(2.0 * (1 << 30) / (ms_c * 1e-3) / 1e9, 1),
            "gemm": "torch.matmul bf16 8192x8192x8192", "copy": "1 GiB read + 1 GiB written"}


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


def per_config(reps=10, wan=None, names=None):
    """Time every configured workload once on the GPU (inputs resident):
    tiny dense + merge, Wan dense + merge, block-sparse at three top-K ratios,
    ragged 12-head, mixed 40-head.  FLOPs are algorithmic (4 d per score of
    every key set attended); kv bytes are the distinct K/V bytes the call
    must read.  `names` restricts the run to those entries (for per-workload
    counter collection); their inputs are still built."""
    import torch
    import kv_cache_attention_chunk_amd as ca
    from kv_cache_attention_chunk_amd import workloads as wl
    want = lambda n: names is None or n in names
    dev = lambda t: torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out = {}

    def merged_fn(q, k, v, w, seg):
        br = []
        for key in ("local_blocks", "history_blocks"):
            blocks = np.array(w.meta[key], np.int32)
            BH = w.B * w.H
            br.append((i32(np.arange(BH + 1) * len(blocks)), i32(np.tile(blocks, BH)),
                       torch.empty((w.B, w.Nq, w.H, w.d), dtype=torch.float32, device="cuda"),
                       torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")))
        om = torch.empty_like(q)
        lm = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

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
    kvb = 2.0 * w.Nkv * w.H * w.d * 2
    if want("tiny_dense"):
        ms_d = _time_ms(torch, lambda: ca.chunk_attn_fwd(q, k, v, scale=w.scale), reps)
        ms_m = _time_ms(torch, merged_fn(q, k, v, w, w.Nkv), reps)
        out["tiny_dense"] = {"dense_us": round(ms_d * 1e3, 1),
                             "local_history_merge_us": round(ms_m * 1e3, 1), "gflop": round(f / 1e9, 3)}
    # Wan-1.3B layer: dense and local/history merge
    w = wan or wl.wan_dense(seed=0)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    f = 4.0 * w.d * w.Nq * w.Nkv * w.B * w.H
    kvb = 2.0 * w.Nkv * w.H * w.d * 2
    if want("wan_dense"):
        out["wan_dense"] = _rec(_time_ms(torch, lambda: ca.chunk_attn_fwd(q, k, v, scale=w.scale), reps),
                                f, kvb)
    # per-call spread, warm (one K/V set, resident in the 256 MB Infinity
    # Cache) and cold (three K/V copies in rotation: 603 MB, more than the
    # Infinity Cache and L2 hold, so each call reads its K/V from HBM)
    if want("wan_dense"):
        o_w = torch.empty_like(q)
        l_w = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        warm = _time_calls(torch, lambda i=0: ca.chunk_attn_fwd(q, k, v, scale=w.scale, out=o_w, lse=l_w),
                           30)
        sets = [(k, v), (k.clone(), v.clone()), (k.clone(), v.clone())]
        cold = _time_calls(torch, lambda i=0: ca.chunk_attn_fwd(
            q, sets[i % 3][0], sets[i % 3][1], scale=w.scale, out=o_w, lse=l_w), 30)
        del sets
        for name, t in (("warm", warm), ("cold", cold)):
            out["wan_dense"][f"{name}_ms_median"] = round(float(np.median(t)), 4)
            out["wan_dense"][f"{name}_ms_min"] = round(float(t.min()), 4)
        out["wan_dense"]["cold_tflops_median"] = round(f / (float(np.median(cold)) * 1e-3) / 1e12, 1)
        out["wan_dense"]["cold_kv_GBs_median"] = round(kvb / (float(np.median(cold)) * 1e-3) / 1e9, 1)
    if want("wan_merge_variant"):
        out["wan_merge_variant"] = _rec(_time_ms(torch, merged_fn(q, k, v, w, 1560), reps), f, kvb)
    # local (sink + chunk frames) and full attention from one pass over each head's list
    row = np.array(w.meta["local_blocks"] + w.meta["history_blocks"], np.int32)
    dip, dix = i32(np.arange(w.B * w.H + 1) * len(row)), i32(np.tile(row, w.B * w.H))
    n_loc = len(w.meta["local_blocks"])
    f_loc = 4.0 * w.d * w.Nq * w.B * w.H * float(_block_len(w.meta["local_blocks"]).sum())
    if want("wan_dual_output"):
        out["wan_dual_output"] = _rec(_time_ms(torch, lambda: ca.chunk_attn_dual_fwd(
            q, k, v, dip, dix, n_loc, kv_block=64, kv_seg=1560, q_block=w.Nq, q_seg=w.Nq,
            scale=w.scale, out_dtype=torch.float32), reps), f, kvb,
            local_gflop_shared=round(f_loc / 1e9, 2))
    # block-sparse path at the three top-K ratios (selection included)
    km = ca.block_mean(k, 64, 1560)
    nqb = ca.num_blocks(w.Nq, 64, 1560)
    qlen = np.tile(_block_len(np.arange(nqb)), w.B * w.H)
    for ratio in (0.25, 0.125, 0.0625):
        lay = wl.sparse_layout(w, ratio)
        if not want(f"sparse_K{lay['K']}"):
            continue
        fn = lambda: ca.block_sparse_fwd(
            q, k, v, sink_begin=0, sink_count=lay["sink_count"], hist_begin=lay["hist_begin"],
            hist_count=lay["hist_count"], C=lay["C"], local_begin=lay["local_begin"],
            local_count=lay["local_count"], K=lay["K"], block=64, seg=1560, k_mean=km,
            scale=w.scale)
        _, _, info = fn()
        torch.cuda.synchronize()
        sp, sx = info["shared_indptr"].cpu().numpy(), info["shared_indices"].cpu().numpy()
        lp, lx = info["local_indptr"].cpu().numpy(), info["local_indices"].cpu().numpy()
        sh = np.array([_block_len(sx[sp[r]:sp[r + 1]]).sum() for r in range(w.B * w.H)])
        lo = np.array([_block_len(lx[lp[r]:lp[r + 1]]).sum() for r in range(w.B * w.H * nqb)])
        f = 4.0 * w.d * (float(sh.sum()) * w.Nq + float((lo * qlen).sum()))
        uniq = sum(_block_len(np.union1d(sx[sp[h]:sp[h + 1]], lx[lp[h * nqb]:lp[(h + 1) * nqb]])).sum()
                   for h in range(w.B * w.H))
        kvb = 2.0 * float(uniq) * w.d * 2
        ms = _time_ms(torch, fn, reps)
        # dense-equivalent rate: the dense layer's FLOPs over the sparse path's time
        f_dense = 4.0 * w.d * w.Nq * w.Nkv * w.B * w.H
        out[f"sparse_K{lay['K']}"] = _rec(ms, f, kvb, ratio=ratio,
                                          dense_equiv_tflops=round(f_dense / (ms * 1e-3) / 1e12, 1))
    # persistent-memory update when the window slides: the chunk's 75 local
    # blocks are evicted into the candidates of each head's 32 persistent blocks
    lay = wl.sparse_layout(w, 0.125)
    _, cm = ca.block_mean(q, 64, 1560, with_total=True)
    pers = ca.block_score_topk(cm, km, lay["C"], cand_begin=lay["hist_begin"],
                               cand_count=lay["hist_count"])[:, :, 0, :].contiguous()
    if want("persistent_update"):
        ms = _time_ms(torch, lambda: ca.persistent_update(cm, km, pers, lay["local_begin"],
                                                          lay["local_count"], lay["C"]), reps)
        out["persistent_update"] = {"us": round(ms * 1e3, 1), "us_median": round(ms.median * 1e3, 1),
                                    "us_min": round(ms.minimum * 1e3, 1), "candidates_per_head":
                                    lay["C"] + lay["local_count"], "C": lay["C"], "heads": w.H}
    del q, k, v, km
    # ragged per-head caches
    w = wl.ragged(seed=0)
    q, kf, vf, cu = dev(w.q), dev(w.k_flat), dev(w.v_flat), i32(w.cu_seqlens)
    tot = int(w.cu_seqlens[-1])
    f = 4.0 * w.d * w.Nq * tot
    kvb = 2.0 * tot * w.d * 2
    if want("ragged"):
        out["ragged"] = _rec(_time_ms(torch, lambda: ca.chunk_attn_varlen_fwd(
            q, kf, vf, cu, cu_seqlens_host=w.cu_seqlens, scale=w.scale), reps), f, kvb,
            sum_len=tot, lengths_frames=w.meta["n_frames"])
    # packing those ragged caches from the dense per-head cache (HBM-bound:
    # every packed K/V row read once and written once)
    kd, vd = dev(w.k), dev(w.v)
    plan = ca.pack_plan([w.ragged_frames[bh] for bh in range(w.B * w.H)], kd.device)
    if want("ragged_pack"):
        ms = _time_ms(torch, lambda: ca.pack_ragged(kd, vd, plan, 1560), reps)
        moved = 2.0 * 2.0 * tot * w.d * 2
        out["ragged_pack"] = {"us": round(ms * 1e3, 1), "us_median": round(ms.median * 1e3, 1),
                              "us_min": round(ms.minimum * 1e3, 1), "bytes_moved_MB": round(moved / 1e6, 1),
                              "GBs": round(moved / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del q, kf, vf, kd, vd
    # latent KV cache (d_c = 192, d_rope = 32): absorbed query, latent
    # attention, per-head up-projection
    m = wl.wan_mla(seed=0)
    mq, mwk, mwv = dev(m["q"]), dev(m["w_uk"]), dev(m["w_uv"])
    mkv = ca.cast_bf16_to_f16(dev(m["kv_lat"]))
    if want("wan_mla"):
        ms_all = _time_ms(torch, lambda: ca.mla_chunk_attn(mq, mkv, mwk, mwv, scale=m["scale"]), reps)
        rows = m["Nq"] * m["H"]
        f_att = 2.0 * rows * m["Nkv"] * (224 + 192)
        f_proj = 2.0 * rows * (96 * 192 + 192 * 128)
        kvb = m["Nkv"] * 224 * 2.0
        out["wan_mla"] = _rec(ms_all, f_att + f_proj, kvb, attention_gflop=round(f_att / 1e9, 1),
                              projection_gflop=round(f_proj / 1e9, 1),
                              kv_bytes_vs_dense=round(kvb / (2.0 * m["Nkv"] * m["H"] * 128 * 2), 4))
    del mq, mwk, mwv, mkv
    # mixed 40-head layer (dense / block lists / ragged per head)
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
    ip = np.zeros(len(lists) + 1, np.int32)
    ip[1:] = np.cumsum([len(x) for x in lists])
    ix = i32(np.concatenate(lists))
    ip = i32(ip)
    kf, vf, cu = dev(w.k_flat), dev(w.v_flat), i32(w.cu_seqlens)
    if want("mixed_40h"):
        out["mixed_40h"] = _rec(_time_ms(torch, lambda: ca.chunk_attn_mixed_fwd(
            q, w.head_mode, k=k, v=v, kv_indptr=ip, kv_indices=ix, kv_block=64, kv_seg=1560,
            q_block=64, q_seg=1560, k_flat=kf, v_flat=vf, cu_seqlens=cu,
            cu_seqlens_host=w.cu_seqlens, scale=w.scale), reps), f, kvb,
            heads_dense_sparse_ragged=[int((w.head_mode == m).sum()) for m in range(3)])
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--topk-ratio", type=float, default=0.125)
    ap.add_argument("--only", choices=["step", "dense", "copy", "configs"], default="step",
                    help="'dense' times the dense kernel alone (for counter runs); 'copy' "
                         "runs a plain 1 GiB device copy, the reference for HBM byte counters")
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

    def sparse():
        return ca.block_sparse_fwd(q, k, v, sink_begin=0, sink_count=lay["sink_count"],
                                   hist_begin=lay["hist_begin"], hist_count=lay["hist_count"],
                                   C=lay["C"], local_begin=lay["local_begin"],
                                   local_count=lay["local_count"], K=lay["K"], block=64,
                                   seg=1560, k_mean=k_mean_resident, scale=w.scale)

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
        out["configs"] = per_config(wan=w)
        roofs = measured_roofs(torch)
        out["measured_roofs"] = roofs
        out["roofline"]["frac_of_measured_gemm"] = round(achieved / roofs["bf16_gemm_tflops"], 4)
        log(f"per-workload timings in {time.perf_counter() - t0:.1f} s")
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f} s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

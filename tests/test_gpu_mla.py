"""GPU parity of chunk attention over a latent KV cache (VideoMLA page,
method): absorbed query, latent attention and per-head up-projection on the
GPU against the CPU oracle, which reconstructs every head's keys and values
from the latent and runs plain attention (O max-abs 1e-2, LSE 1e-3)."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_chunk_amd as ca
import oracle as orc
from kv_cache_attention_chunk_amd import workloads as wl
from helpers import assert_lse, assert_o, assert_written, nan_lse, nan_out, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _bf(rng, shape, scale=1.0):
    return wl.Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32) * scale)


def _run(q, kv, wk, wv, scale, out_dtype=torch.bfloat16):
    kv16 = ca.cast_bf16_to_f16(to_dev(kv))
    return ca.mla_chunk_attn(to_dev(q), kv16, to_dev(wk), to_dev(wv), scale=scale, out_dtype=out_dtype)


def _ref(q, kv, wk, wv, scale, rows=None, heads=None):
    return orc.mla_chunk_attn(q.f32, kv.f32[..., :192], kv.f32[..., 192:], wk.f32, wv.f32, scale,
                              rows=rows, heads=heads)


def test_cast_bf16_to_f16_rounds_to_nearest_even():
    say("bf16 -> fp16 cast")
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096).astype(np.float32) * np.exp2(rng.integers(-20, 12, 4096)).astype(np.float32)
    xb = wl.Bf16Tensor.from_f32(x)
    y = ca.cast_bf16_to_f16(to_dev(xb))
    torch.cuda.synchronize()
    ref = xb.f32.astype(np.float16)              # IEEE round to nearest even
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_cast_bf16_to_f16_saturates_beyond_fp16_range():
    say("bf16 -> fp16 cast: saturation and NaN")
    x = np.array([65504.0, 65536.0, -70000.0, 3.0e38, -3.0e38, np.inf, -np.inf, np.nan,
                  1.0e-6, -2.0e-8, 0.0, -0.0, 1.5, 65280.0, -65280.0, 6.0e-5], np.float32)
    xb = wl.Bf16Tensor.from_f32(x)
    y = ca.cast_bf16_to_f16(to_dev(xb)).cpu().numpy()
    torch.cuda.synchronize()
    xr = xb.f32
    ref = np.clip(xr, -65504.0, 65504.0).astype(np.float16)   # NaN stays NaN
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(y[fin].view(np.uint16), ref[fin].view(np.uint16))
    assert np.all(np.isfinite(y[fin]))


@pytest.mark.parametrize("B,Nq,H,N,out_dtype", [
    (2, 70, 3, 150, torch.bfloat16),     # partial key tile, partial row tile
    (1, 33, 5, 64, torch.float32),       # one full tile
    (1, 1, 2, 1000, torch.float32),      # one query, many tiles
])
def test_mla_small(B, Nq, H, N, out_dtype):
    say(f"mla B={B} Nq={Nq} H={H} N={N}")
    rng = np.random.default_rng(N + H)
    q, kv = _bf(rng, (B, Nq, H, 128), 1.5), _bf(rng, (B, N, 224))
    wk, wv = _bf(rng, (H, 96, 192), 1 / math.sqrt(192)), _bf(rng, (H, 128, 192), 1 / math.sqrt(192))
    o, l, _ = _run(q, kv, wk, wv, 1 / math.sqrt(128), out_dtype)
    torch.cuda.synchronize()
    Or, Lr = _ref(q, kv, wk, wv, 1 / math.sqrt(128))
    assert_o(o, Or, out_dtype == torch.bfloat16, "mla")
    assert_lse(l, Lr, "mla")


def test_mla_empty_cache():
    say("mla empty cache")
    rng = np.random.default_rng(3)
    q = _bf(rng, (1, 20, 2, 128))
    kv = torch.zeros((1, 0, 224), dtype=torch.float16, device="cuda")
    wk, wv = _bf(rng, (2, 96, 192)), _bf(rng, (2, 128, 192))
    o, l, _ = ca.mla_chunk_attn(to_dev(q), kv, to_dev(wk), to_dev(wv))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_mla_wan_shape():
    say("mla wan shape: 12 heads x 4680 queries vs 32760 latent rows")
    w = wl.wan_mla(seed=0)
    B, Nq, H = 1, w["q"].shape[1], w["q"].shape[2]
    o, l = nan_out(B, Nq, H, 128), nan_lse(B, H, Nq)
    o_lat = torch.full((B, Nq, H, 192), float("nan"), dtype=torch.float32, device="cuda")
    kv16 = ca.cast_bf16_to_f16(to_dev(w["kv_lat"]))
    ca.mla_chunk_attn(to_dev(w["q"]), kv16, to_dev(w["w_uk"]), to_dev(w["w_uv"]),
                      scale=w["scale"], out=o, lse=l, o_lat=o_lat)
    torch.cuda.synchronize()
    assert_written("mla wan", o, l, o_lat)
    # a (query, head) row of every 32-row wave slice: kernel rows are the
    # flattened (query, head) pairs n * H + h
    rng = np.random.default_rng(6)
    flat = [int(rng.integers(s, min(s + 32, Nq * H))) for s in range(0, Nq * H, 32)]
    by_head = {}
    for r in flat:
        by_head.setdefault(r % H, []).append(r // H)
    og, lg = o.float().cpu().numpy(), l.cpu().numpy()
    for h, rows in sorted(by_head.items()):
        rows = np.array(sorted(set(rows)))
        Or, Lr = _ref(w["q"], w["kv_lat"], w["w_uk"], w["w_uv"], w["scale"], rows=rows,
                      heads=[h])
        assert_o(og[:, rows, h:h + 1], Or, True, f"mla wan head {h}")
        assert_lse(lg[:, h:h + 1, rows], Lr, f"mla wan head {h}")

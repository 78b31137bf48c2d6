"""Seeded synthetic inputs for chunk attention over a video-generation KV cache.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic (no attention, no pooling, no scoring, no selection).  The
CPU oracle and the HIP path both consume what it returns.  It imports numpy
only, so loading it never touches the GPU library.

Shapes follow the pages' workloads:
  * Wan-1.3B self-attention: 12 heads x 128 dims (VideoMLA page, problem
    statement and the "12 x 128 = 1536" example).
  * one latent frame = 1560 tokens, a 21-frame sliding-window KV cache
    (VideoMLA page, problem statement: the ~6.0 GB figure for 21 frames).
  * a new chunk = 3 latent frames whose K/V are the newest 3 frames of the
    cache (Sparse Forcing page, section 2.1 local window).
  * ragged per-head caches: sink frame + forced recent frames + a per-head
    subset of the middle frames chosen by a stride, periodic or recent-window
    rule (Pyramid Forcing page, section 2 cache policies and section 3 ragged
    cache), flattened head after head with cu_seqlens boundaries.

bf16 tensors are produced as uint16 bit patterns (round-to-nearest-even of
float32 standard normals) together with their exact float32 values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

FRAME_TOKENS = 1560          # tokens per latent frame (Wan-1.3B latent grid)
CACHE_FRAMES = 21            # sliding-window cache length in frames
CHUNK_FRAMES = 3             # frames per generated chunk
BLOCK_TOKENS = 64            # spatio-temporal block size used for selection


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> exactly equal float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Bf16Tensor:
    """A bf16 tensor kept both as raw bits and as its exact float32 value
    (computed once, on first use)."""
    bits: np.ndarray
    _f32: Optional[np.ndarray] = dataclasses.field(default=None, repr=False, compare=False)

    @property
    def f32(self) -> np.ndarray:
        if self._f32 is None:
            self._f32 = bf16_to_f32(self.bits)
        return self._f32

    @property
    def shape(self):
        return self.bits.shape

    @staticmethod
    def from_f32(x: np.ndarray) -> "Bf16Tensor":
        return Bf16Tensor(bf16_bits(x))


def _normal_bf16(rng: np.random.Generator, shape) -> Bf16Tensor:
    return Bf16Tensor.from_f32(rng.standard_normal(shape, dtype=np.float32))


def ragged_frame_subset(head_class: int, n_frames: int,
                        first_mid: int = 1, last_mid: int = 18) -> List[int]:
    """Frames held by one ragged head: sink frame 0, the middle frames the
    head's policy keeps, and the forced recent frames.

    n_frames counts all frames the head keeps (3..21 for a 21-frame cache).
    The three fixed frames are the sink (frame 0) and the two newest frames
    (19, 20); the remaining n_frames - 3 slots come from frames
    first_mid..last_mid according to the head class:
      0 anchor: evenly spaced over the middle range (adaptive stride),
      1 wave:   every P-th frame going back from last_mid (periodic sampling),
      2 veil:   the most recent contiguous middle frames (recent window).
    """
    m = n_frames - 3
    span = last_mid - first_mid + 1
    if not 0 <= m <= span:
        raise ValueError(f"n_frames={n_frames} out of range")
    if m == 0:
        mid: List[int] = []
    elif head_class == 0:
        mid = sorted({int(round(x)) for x in np.linspace(first_mid, last_mid, m)})
    elif head_class == 1:
        period = max(1, span // m)
        mid = sorted(last_mid - j * period for j in range(m))
    elif head_class == 2:
        mid = list(range(last_mid - m + 1, last_mid + 1))
    else:
        raise ValueError("head_class must be 0, 1 or 2")
    assert len(mid) == m and len(set(mid)) == m
    return [0] + mid + [last_mid + 1, last_mid + 2]


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    d: int
    Nq: int
    Nkv: int
    q: Bf16Tensor                      # [B, Nq, H, d]
    k: Optional[Bf16Tensor]            # [B, Nkv, H, d] dense cache
    v: Optional[Bf16Tensor]
    scale: float
    head_scale: Optional[np.ndarray] = None
    # block tiling of the KV axis and the query axis (block size, segment)
    kv_block: int = BLOCK_TOKENS
    kv_seg: int = FRAME_TOKENS
    q_block: int = BLOCK_TOKENS
    q_seg: int = FRAME_TOKENS
    # ragged per-head caches
    k_flat: Optional[Bf16Tensor] = None    # [total, d]
    v_flat: Optional[Bf16Tensor] = None
    cu_seqlens: Optional[np.ndarray] = None  # int32 [B*H + 1]
    ragged_frames: Optional[Dict[int, List[int]]] = None  # bh -> frames
    # per-head mode for the mixed workload: 0 dense, 1 block-sparse, 2 ragged
    head_mode: Optional[np.ndarray] = None
    meta: Dict = dataclasses.field(default_factory=dict)


def _flatten_ragged(k: Bf16Tensor, v: Bf16Tensor, frames_per_bh: Dict[int, List[int]],
                    B: int, H: int, frame_tokens: int):
    """Copy each listed (b, h)'s frames out of a dense cache into one flat
    [total, d] buffer, head after head; heads not listed get length 0."""
    lens = np.zeros(B * H, dtype=np.int64)
    for bh, fr in frames_per_bh.items():
        lens[bh] = len(fr) * frame_tokens
    cu = np.zeros(B * H + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    d = k.bits.shape[-1]
    kf = np.empty((int(cu[-1]), d), dtype=np.uint16)
    vf = np.empty((int(cu[-1]), d), dtype=np.uint16)
    for bh, fr in frames_per_bh.items():
        b, h = divmod(bh, H)
        pos = int(cu[bh])
        for f in fr:
            sl = slice(f * frame_tokens, (f + 1) * frame_tokens)
            kf[pos:pos + frame_tokens] = k.bits[b, sl, h, :]
            vf[pos:pos + frame_tokens] = v.bits[b, sl, h, :]
            pos += frame_tokens
    return Bf16Tensor(kf), Bf16Tensor(vf), cu.astype(np.int32)


def tiny_dense(seed: int = 0, B: int = 1, H: int = 2, d: int = 64,
               Nq: int = 256, Nkv: int = 1024, sink: int = 64) -> Workload:
    """Tiny dense chunk: 256 queries vs 1024 cached tokens (64 sink + 960),
    the chunk's own K/V being the last 256 cache tokens.  Flat 64-token block
    tiling (one segment), so local = sink block + the chunk's blocks."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, Nq, H, d))
    k = _normal_bf16(rng, (B, Nkv, H, d))
    v = _normal_bf16(rng, (B, Nkv, H, d))
    nblk = Nkv // BLOCK_TOKENS
    local = list(range(sink // BLOCK_TOKENS)) + list(range((Nkv - Nq) // BLOCK_TOKENS, nblk))
    history = [b for b in range(nblk) if b not in local]
    return Workload("tiny_dense", B, H, d, Nq, Nkv, q, k, v, 1.0 / np.sqrt(d),
                    kv_block=BLOCK_TOKENS, kv_seg=Nkv, q_block=BLOCK_TOKENS, q_seg=Nq,
                    meta={"local_blocks": local, "history_blocks": history, "seed": seed})


def wan_dense(seed: int = 0, H: int = 12, d: int = 128, frames_q: int = CHUNK_FRAMES,
              frames_kv: int = CACHE_FRAMES, frame_tokens: int = FRAME_TOKENS,
              head_scales: bool = True) -> Workload:
    """Wan-1.3B-shaped layer: 3-frame query chunk vs 21-frame cache, bf16
    N(0,1); each head's Q and K multiplied by s_h ~ U[0.5, 2]."""
    B = 1
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.5, 2.0, size=H).astype(np.float32) if head_scales else None
    Nq, Nkv = frames_q * frame_tokens, frames_kv * frame_tokens
    qf = rng.standard_normal((B, Nq, H, d), dtype=np.float32)
    kf = rng.standard_normal((B, Nkv, H, d), dtype=np.float32)
    if s is not None:
        qf *= s[None, None, :, None]
        kf *= s[None, None, :, None]
    q = Bf16Tensor.from_f32(qf)
    del qf
    k = Bf16Tensor.from_f32(kf)
    del kf
    v = _normal_bf16(rng, (B, Nkv, H, d))
    bpf = -(-frame_tokens // BLOCK_TOKENS)
    sink_frames = [0]
    chunk_frames = list(range(frames_kv - frames_q, frames_kv))
    local_frames = sink_frames + chunk_frames
    blocks = lambda frs: [f * bpf + j for f in frs for j in range(bpf)]
    hist_frames = [f for f in range(frames_kv) if f not in local_frames]
    return Workload("wan_dense", B, H, d, Nq, Nkv, q, k, v, 1.0 / np.sqrt(d),
                    head_scale=s, kv_seg=frame_tokens, q_seg=frame_tokens,
                    meta={"local_blocks": blocks(local_frames),
                          "history_blocks": blocks(hist_frames),
                          "blocks_per_frame": bpf, "frames_kv": frames_kv,
                          "frames_q": frames_q, "seed": seed})


def sparse_layout(w: Workload, topk_ratio: float, persistent: int = 32) -> Dict:
    """Block-sparse layout on a frame-aligned workload: sink frame blocks,
    history blocks (persistent candidates) and local-window blocks (top-K
    candidates = the chunk's own frames), K = ceil(ratio * local blocks)."""
    bpf = -(-w.kv_seg // w.kv_block)
    frames_kv = w.Nkv // w.kv_seg
    frames_q = w.Nq // w.q_seg
    local_begin = (frames_kv - frames_q) * bpf
    n_local = frames_q * bpf
    return {"sink_begin": 0, "sink_count": bpf,
            "hist_begin": bpf, "hist_count": local_begin - bpf,
            "local_begin": local_begin, "local_count": n_local,
            "C": persistent, "K": int(np.ceil(topk_ratio * n_local - 1e-9)),
            "ratio": topk_ratio}


def ragged(seed: int = 0, H: int = 12, d: int = 128, frames_q: int = CHUNK_FRAMES,
           frames_kv: int = CACHE_FRAMES, frame_tokens: int = FRAME_TOKENS) -> Workload:
    """Ragged per-head caches: head h keeps n_h ~ U{3..21} frames (sink +
    policy-chosen middle frames + 2 forced recent frames); the policy is
    h mod 3 (stride / periodic / recent window).  Frame contents come from a
    per-head dense N(0,1) cache, so every head's data stays N(0,1)."""
    B = 1
    rng = np.random.default_rng(seed)
    Nq, Nkv = frames_q * frame_tokens, frames_kv * frame_tokens
    q = _normal_bf16(rng, (B, Nq, H, d))
    k = _normal_bf16(rng, (B, Nkv, H, d))
    v = _normal_bf16(rng, (B, Nkv, H, d))
    n = rng.integers(3, frames_kv + 1, size=B * H)
    frames = {bh: ragged_frame_subset((bh % H) % 3, int(n[bh]), 1, frames_kv - 3)
              for bh in range(B * H)}
    kf, vf, cu = _flatten_ragged(k, v, frames, B, H, frame_tokens)
    return Workload("ragged", B, H, d, Nq, Nkv, q, k, v, 1.0 / np.sqrt(d),
                    kv_seg=frame_tokens, q_seg=frame_tokens,
                    k_flat=kf, v_flat=vf, cu_seqlens=cu, ragged_frames=frames,
                    meta={"n_frames": n.tolist(), "seed": seed})


def mixed(seed: int = 0, H: int = 40, d: int = 128, frames_q: int = CHUNK_FRAMES,
          frames_kv: int = CACHE_FRAMES, frame_tokens: int = FRAME_TOKENS,
          topk_ratio: float = 0.125) -> Workload:
    """14B-class layer with per-head modes h mod 3 -> dense / block-sparse /
    ragged.  All heads share one dense [1, Nkv, H, d] cache; ragged heads
    additionally get their frame subset flattened (policy = (h // 3) mod 3)."""
    B = 1
    rng = np.random.default_rng(seed)
    Nq, Nkv = frames_q * frame_tokens, frames_kv * frame_tokens
    q = _normal_bf16(rng, (B, Nq, H, d))
    k = _normal_bf16(rng, (B, Nkv, H, d))
    v = _normal_bf16(rng, (B, Nkv, H, d))
    mode = np.array([h % 3 for h in range(H)], dtype=np.int32)
    n = rng.integers(3, frames_kv + 1, size=H)
    frames = {h: ragged_frame_subset((h // 3) % 3, int(n[h]), 1, frames_kv - 3)
              for h in range(H) if mode[h] == 2}
    kf, vf, cu = _flatten_ragged(k, v, frames, B, H, frame_tokens)
    w = Workload("mixed", B, H, d, Nq, Nkv, q, k, v, 1.0 / np.sqrt(d),
                 kv_seg=frame_tokens, q_seg=frame_tokens,
                 k_flat=kf, v_flat=vf, cu_seqlens=cu, ragged_frames=frames,
                 head_mode=mode, meta={"n_frames": n.tolist(), "seed": seed})
    w.meta["sparse"] = sparse_layout(w, topk_ratio)
    return w


def wan_mla(seed: int = 0, H: int = 12, d_nope: int = 96, d_rope: int = 32, d_c: int = 192,
            d_v: int = 128, frames_q: int = CHUNK_FRAMES, frames_kv: int = CACHE_FRAMES,
            frame_tokens: int = FRAME_TOKENS) -> Dict:
    """Latent-KV (VideoMLA page, method) layer at the Wan-1.3B shape: per
    token a shared content latent (d_c = 192) and one shared rotated position
    key (d_rope = 32) -- 224 cached values per token instead of 2 x 12 x 128 --
    and per-head up-projections.  bf16 N(0,1) queries, latents and position
    keys; random up-projections N(0, 1/d_c), so reconstructed keys and values
    have unit variance (no trained weights exist here; they are not needed
    for kernel parity).  The latent cache is one [B, N, d_c + d_rope] array
    (content latent first); `c_kv` and `k_rope` are its two column ranges."""
    B = 1
    rng = np.random.default_rng(seed)
    Nq, Nkv = frames_q * frame_tokens, frames_kv * frame_tokens
    q = _normal_bf16(rng, (B, Nq, H, d_nope + d_rope))
    kv_lat = _normal_bf16(rng, (B, Nkv, d_c + d_rope))
    w_uk = Bf16Tensor.from_f32(rng.standard_normal((H, d_nope, d_c), dtype=np.float32) / np.sqrt(d_c))
    w_uv = Bf16Tensor.from_f32(rng.standard_normal((H, d_v, d_c), dtype=np.float32) / np.sqrt(d_c))
    return {"B": B, "H": H, "Nq": Nq, "Nkv": Nkv, "d_nope": d_nope, "d_rope": d_rope,
            "d_c": d_c, "d_v": d_v, "q": q, "kv_lat": kv_lat, "w_uk": w_uk, "w_uv": w_uv,
            "scale": 1.0 / np.sqrt(d_nope + d_rope), "seed": seed}


def kv_cache_bytes(H: int, d: int, tokens: int, layers: int, elem_bytes: int = 2) -> int:
    """Bytes of a per-head dense K+V cache for `layers` layers."""
    return 2 * H * d * elem_bytes * tokens * layers


def random_csr(rng: np.random.Generator, rows: int, n_blocks: int, max_per_row: int,
               allow_empty: bool = True):
    """Random sorted, unique block lists (CSR) for parity tests."""
    lists = []
    for _ in range(rows):
        lo = 0 if allow_empty else 1
        m = int(rng.integers(lo, max_per_row + 1))
        lists.append(np.sort(rng.choice(n_blocks, size=min(m, n_blocks), replace=False)))
    indptr = np.zeros(rows + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(x) for x in lists])
    indices = (np.concatenate(lists) if indptr[-1] else np.zeros(0)).astype(np.int32)
    return indptr, indices

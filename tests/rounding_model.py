"""A CPU model of the rounding steps of the attention kernel's arithmetic, used
only to search for inputs on which the bf16-output bar is tight (test
infrastructure; it shares nothing with the HIP library and is not the
oracle).  The modelled steps: float32 scores of bf16 operands, exponent base
= the exact row max, weights p = 2^(s c - m) in float32, p rounded to bf16
for the P.V product (round to nearest even), the row sum l from the float32
weights, O = bf16(acc / l).

The inputs of a trial are drawn from numpy's generator seeded with
[seed, trial], so a case found by the search is reproduced from its two
numbers alone: one query row, n ~ U{2..64} keys, d = 128, Q and K scaled by
s ~ U[0.5, 2] (the per-head scale range of the Wan-shaped workload), V
N(0, 1), all rounded to bf16.
"""
import numpy as np

LOG2E = 1.4426950408889634


def bf16_round(x):
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32)


def trial_inputs(seed, trial, d=128):
    rng = np.random.default_rng([seed, trial])
    n = int(rng.integers(2, 65))
    s = float(rng.uniform(0.5, 2.0))
    q = bf16_round(rng.standard_normal(d).astype(np.float32) * s)
    K = bf16_round(rng.standard_normal((n, d)).astype(np.float32) * s)
    V = bf16_round(rng.standard_normal((n, d)).astype(np.float32))
    return q, K, V


def kernel_model(q, K, V, scale):
    """(O, LSE) of one query row as the kernel rounds them."""
    s = (K.astype(np.float32) @ q.astype(np.float32)).astype(np.float32)
    c = np.float32(scale * LOG2E)
    m = np.float32(s.max() * c)
    p = np.exp2((s * c - m).astype(np.float32)).astype(np.float32)
    acc = (bf16_round(p)[:, None] * V).astype(np.float32).sum(axis=0, dtype=np.float32)
    l = np.float32(p.sum(dtype=np.float32))
    o = bf16_round(acc * np.float32(1.0 / l))
    return o, float((m + np.log2(l)) * np.float32(np.log(2.0)))


# Cases found by searching 320,000 trials (seeds 1-8, trials 0-39,999):
# (seed, trial) -> what makes each one tight (error, |O_ref|, keys).
TIGHT_CASES = {
    (6, 6444): "largest error relative to the bar: 0.0079 at |O_ref| = 1.24, 2 keys",
    (2, 3860): "largest error in [2, 4): 0.0111 at |O_ref| = 2.04, above 1e-2, 2 keys",
    (1, 11154): "0.0107 at |O_ref| = 2.08, above 1e-2, 8 keys",
    (2, 28635): "largest error: 0.0155 at |O_ref| = 4.92, 2 keys",
}


# --------------------------------------------------------------------------
# latent-KV path: the absorbed query is rounded to fp16 for the score MFMA
# --------------------------------------------------------------------------
def f16_round(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def mla_trial_inputs(seed, trial):
    """One query row of one head against n ~ U{1..8} latent rows: q bf16 [128]
    scaled by s ~ U[0.5, 2], latent rows bf16 [n, 224] N(0, 1), W^K bf16
    [96, 192] N(0, 1/192)."""
    rng = np.random.default_rng([seed, trial])
    n = int(rng.integers(1, 9))
    s = float(rng.uniform(0.5, 2.0))
    q = bf16_round(rng.standard_normal(128).astype(np.float32) * s)
    kv = bf16_round(rng.standard_normal((n, 224)).astype(np.float32))
    wk = bf16_round(rng.standard_normal((96, 192)).astype(np.float32) / np.sqrt(192.0))
    return q, kv, wk


def mla_lse_model(q, kv, wk, scale, corrected):
    """LSE of one latent-attention row as the kernel forms it: the absorbed
    query [(W^K)^T q^nope ; q^R] summed in float32 and rounded to fp16; with
    `corrected`, plus scale * (residual . weighted mean latent content row),
    the residual kept to bf16 precision."""
    q_c = (q[:96].astype(np.float64) @ wk.astype(np.float64)).astype(np.float32)
    q16 = np.concatenate([f16_round(q_c), f16_round(q[96:])]).astype(np.float64)
    s = scale * (kv.astype(np.float64) @ q16)
    m = s.max()
    w = np.exp(s - m)
    lse = m + np.log(w.sum())
    if corrected:
        res = bf16_round(q_c - f16_round(q_c)).astype(np.float64)
        o_c = (w / w.sum()) @ kv[:, :192].astype(np.float64)
        lse += scale * float(res @ o_c)
    return float(lse)


# Cases found by searching 200,000 trials (seeds 1-8, trials 0-24,999): the
# uncorrected LSE error of each; the corrected one stays below 2.2e-6 on all.
MLA_TIGHT_CASES = {
    (8, 17715): "uncorrected LSE error 1.59e-3 (2 latent rows)",
    (7, 10682): "uncorrected LSE error 1.34e-3 (3 latent rows)",
    (6, 15334): "uncorrected LSE error 1.32e-3 (1 latent row)",
}

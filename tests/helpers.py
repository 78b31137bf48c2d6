"""Shared helpers of the GPU parity tests: moving generator output to the GPU
and the parity bars (O max-abs 1e-2, LSE max-abs 1e-3, exact block ids
except at near-ties)."""
import numpy as np
import torch

O_TOL = 1e-2
LSE_TOL = 1e-3
TIE_EPS = 1e-4


def to_dev(bf):
    """Bf16Tensor -> torch.bfloat16 on cuda:0 (bit-exact)."""
    return torch.from_numpy(bf.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def o_bound(ref, out_bf16: bool):
    """Allowed |O_gpu - O_ref|: 1e-2, plus the bf16 rounding of the stored
    output where half a bf16 ulp alone exceeds the budget (|O| >= 4)."""
    ref = np.abs(ref)
    b = np.full(ref.shape, O_TOL)
    if out_bf16:
        b = np.where(ref >= 4.0, O_TOL + ref * 2.0 ** -8, b)
    return b


def assert_o(o_gpu, o_ref, out_bf16=True, what=""):
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    assert og.shape == o_ref.shape, (og.shape, o_ref.shape)
    assert np.all(np.isfinite(og)), f"{what}: non-finite O"
    err = np.abs(og - o_ref)
    bound = o_bound(o_ref, out_bf16)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} O elements off, max err {err.max():.3g}"
    return float(err.max())


def assert_lse(l_gpu, l_ref, what=""):
    lg = l_gpu.cpu().numpy().astype(np.float64)
    assert lg.shape == l_ref.shape, (lg.shape, l_ref.shape)
    ninf_ref = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), ninf_ref), f"{what}: -inf pattern differs"
    fin = ~ninf_ref
    err = np.abs(lg[fin] - l_ref[fin]) if fin.any() else np.zeros(1)
    assert err.max() <= LSE_TOL, f"{what}: LSE max err {err.max():.3g}"
    return float(err.max())


def compare_topk(idx_gpu, ref, tie_eps=TIE_EPS):
    """Ids must match exactly except for (b, h, qb) rows whose K-th/(K+1)-th
    score gap is below tie_eps; those may differ only among the near-tied
    candidates.  Returns the number of rows that differed (all at ties)."""
    ig = idx_gpu.cpu().numpy()
    ir = ref["idx"]
    assert ig.shape == ir.shape
    diff = np.any(ig != ir, axis=-1)
    for pos in zip(*np.nonzero(diff)):
        assert ref["gap"][pos] < tie_eps, f"top-K mismatch at {pos} with gap {ref['gap'][pos]}"
    for pos in np.ndindex(ig.shape[:-1]):
        row = ig[pos]
        assert np.all(np.diff(row) > 0), f"ids not ascending/unique at {pos}"
    return int(diff.sum())

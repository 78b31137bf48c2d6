"""The top-K comparison used by the GPU tests, checked on the CPU against
planted selections (CPU only): a selection that differs from the oracle's
only inside the tie band passes; one that drops an id above the band or
takes one below it fails."""
import numpy as np
import pytest

from oracle import chunk_attention as oc
from helpers import compare_topk


def _ref():
    d = 4
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 8, d), np.float32)
    # candidates 0..7 with scores: two near-tied at the K-th place (K = 3)
    k[0, 0, :, 0] = [5.0, 1.0, 3.00002, 3.0, 0.5, 4.0, 2.0, -1.0]
    return oc.block_score_topk(q, k, 0, 8, 3)


def test_exact_and_tie_band_swaps_pass():
    ref = _ref()
    assert ref["idx"][0, 0, 0].tolist() == [0, 2, 5]
    assert ref["gap"][0, 0, 0] < 1e-4
    rep = {}
    assert compare_topk(ref["idx"].copy(), ref, report=rep) == 0
    swapped = ref["idx"].copy()
    swapped[0, 0, 0] = [0, 3, 5]          # block 3 is inside the tie band
    assert compare_topk(swapped, ref, report=rep) == 1
    assert rep["near_tie_rows"] == 2 and rep["rows_differing_at_ties"] == 1


@pytest.mark.parametrize("bad", [[0, 2, 3], [2, 3, 5], [0, 5, 6], [0, 2, 2], [5, 2, 0]])
def test_selections_outside_the_band_fail(bad):
    ref = _ref()
    got = ref["idx"].copy()
    got[0, 0, 0] = bad
    with pytest.raises(AssertionError):
        compare_topk(got, ref)


def test_mismatch_without_a_tie_fails():
    ref = _ref()
    ref["gap"][...] = 1.0                 # pretend the row is not near-tied
    got = ref["idx"].copy()
    got[0, 0, 0] = [0, 3, 5]
    with pytest.raises(AssertionError):
        compare_topk(got, ref)

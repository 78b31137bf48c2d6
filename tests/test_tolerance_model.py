"""Why the parity bars are what they are (CPU only).

A model of the attention kernel's rounding steps (tests/rounding_model.py)
is run on the tightest cases a 320,000-trial search found, against the
oracle:

* bf16 output.  The kernel rounds P to bf16 for the P.V product and rounds
  the output itself to bf16.  Below |O| = 2 the two stay inside 1e-2; from
  |O| = 2 on, half an output ulp alone is 0.0078 (in [2, 4)), so the modelled
  error can pass 1e-2 while staying inside 1e-2 + half an ulp, the bar the
  GPU tests apply (helpers.o_bound).  Float32 outputs carry no output
  rounding and meet 1e-2 everywhere.
* latent-KV LSE.  Rounding the absorbed query to fp16 puts up to 2^-12
  relative error on every score, which moves the LSE past 1e-3 on rows with
  few latent rows; the kernel's first-order correction (scale times the
  rounding residual dotted with the weighted mean latent row) brings it to
  float32 grade.
"""
import numpy as np
import pytest

from oracle import chunk_attention as oc
from helpers import LSE_TOL, O_TOL, o_bound
from rounding_model import (MLA_TIGHT_CASES, TIGHT_CASES, kernel_model, mla_lse_model,
                            mla_trial_inputs, trial_inputs)

SCALE = 1.0 / np.sqrt(128.0)


@pytest.mark.parametrize("case", sorted(TIGHT_CASES))
def test_bf16_output_tight_cases_meet_the_derived_bar(case):
    q, K, V = trial_inputs(*case)
    o, _ = kernel_model(q, K, V, SCALE)
    O, _ = oc.attention(q[None], K, V, SCALE)
    err = np.abs(o.astype(np.float64) - O[0])
    assert np.all(err <= o_bound(O[0], True)), TIGHT_CASES[case]


def test_the_output_half_ulp_is_needed_in_2_to_4():
    """The plain 1e-2 bar fails the model on a row with |O_ref| in [2, 4):
    the relaxation is needed there, and it is the output's own rounding."""
    q, K, V = trial_inputs(2, 3860)
    o, _ = kernel_model(q, K, V, SCALE)
    O, _ = oc.attention(q[None], K, V, SCALE)
    err = np.abs(o.astype(np.float64) - O[0])
    i = int(err.argmax())
    assert err[i] > O_TOL and 2.0 <= abs(O[0, i]) < 4.0
    # the float32 value before the output rounding meets 1e-2
    s = (K @ q).astype(np.float32)
    c = np.float32(SCALE * 1.4426950408889634)
    p = np.exp2((s * c - np.float32(s.max() * c)).astype(np.float32))
    from rounding_model import bf16_round
    acc = (bf16_round(p)[:, None] * V).astype(np.float32).sum(axis=0, dtype=np.float32)
    o32 = acc * np.float32(1.0 / np.float32(p.sum(dtype=np.float32)))
    assert np.abs(o32.astype(np.float64) - O[0]).max() <= O_TOL


@pytest.mark.parametrize("case", sorted(MLA_TIGHT_CASES))
def test_latent_lse_correction(case):
    q, kv, wk = mla_trial_inputs(*case)
    _, L = oc.mla_chunk_attn(q[None, None, None, :], kv[None, :, :192], kv[None, :, 192:],
                             wk[None], np.zeros((1, 128, 192)), SCALE)
    plain = abs(mla_lse_model(q, kv, wk, SCALE, False) - L[0, 0, 0])
    fixed = abs(mla_lse_model(q, kv, wk, SCALE, True) - L[0, 0, 0])
    assert plain > LSE_TOL, MLA_TIGHT_CASES[case]     # the fp16 query alone misses 1e-3
    assert fixed < 1e-5                                # the corrected LSE is float32-grade

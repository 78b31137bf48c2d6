"""The benchmark's host-side helpers, checked on the CPU: the parity-sample
rows cover every 32-row wave slice of every workgroup; the CPU leg's O/LSE
statistics classify errors against the bars as the GPU tests do; its top-K
statistics count differing rows and tell tie-band differences from real
ones; the cold-rotation copy count; the counter summaries attach only to the
code they were taken on."""
import json
import os

import numpy as np
import pytest

import bench
from oracle import chunk_attention as oc


def test_sample_rows_cover_every_wave_slice():
    Nq = 4680
    rows = bench._sample_rows(Nq, 64, 1560, seed=1)
    assert rows[0] == 0 and rows[-1] == Nq - 1 and np.all(np.diff(rows) > 0)
    # every 32-row slice of the 256-row query tiles holds a sampled row
    assert set(np.unique(rows // 32)) == set(range(-(-Nq // 32)))
    # every 32-row slice of every 64-token query block (frame-aligned tiling)
    spans = oc.block_spans(Nq, 64, 1560)
    for s, ln in spans:
        for o in range(0, ln, 32):
            lo, hi = s + o, s + min(o + 32, ln)
            assert np.any((rows >= lo) & (rows < hi)), (s, ln, o)
    # without a block tiling only the tile slices are required
    r2 = bench._sample_rows(1000, seed=3)
    assert set(np.unique(r2 // 32)) == set(range(-(-1000 // 32)))


def test_o_stats_bars():
    ref = np.array([0.5, -1.9, 2.5, 3.0, -6.0])
    # errors: inside 1e-2; just below 1e-2; within 1e-2 + half-ulp(2.5) = 1e-2 + 2^-7;
    # beyond it; and at |O| = 6 within 1e-2 + 2^-6
    err = np.array([0.004, 0.0099, 0.0105, 0.0190, 0.025])
    st = bench._o_stats(ref + err, ref, True)
    assert st["o_elements"] == 5
    assert st["o_relaxed_bound"] == 2          # 2.5 and 6.0
    assert st["o_over_bar"] == 1               # 3.0: 0.019 > 1e-2 + 2^-7
    assert abs(st["max_abs_dO"] - 0.025) < 1e-12
    # a float32 output gets no relaxation
    st32 = bench._o_stats(ref + err, ref, False)
    assert st32["o_relaxed_bound"] == 0 and st32["o_over_bar"] == 3
    # a NaN (an unwritten output) counts as beyond the bar
    bad = ref.copy()
    bad[0] = np.nan
    assert bench._o_stats(bad, ref, True)["o_over_bar"] == 1


def test_lse_stats():
    ref = np.array([1.0, -np.inf, 3.0])
    st = bench._lse_stats(np.array([1.0005, -np.inf, 3.002]), ref)
    assert st["lse_over_bar"] == 1 and st["lse_neginf_match"]
    assert abs(st["max_abs_dLSE"] - 0.002) < 1e-9
    assert not bench._lse_stats(np.array([1.0, 0.0, 3.0]), ref)["lse_neginf_match"]


def _ref():
    q = np.zeros((1, 1, 1, 4), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 8, 4), np.float32)
    k[0, 0, :, 0] = [5.0, 1.0, 3.00002, 3.0, 0.5, 4.0, 2.0, -1.0]   # a near-tie at K = 3
    return oc.block_score_topk(q, k, 0, 8, 3)


def test_topk_stats():
    ref = _ref()
    st = bench._topk_stats(ref["idx"], ref)
    assert st == {"rows": 1, "rows_differing": 0, "rows_differing_outside_tie_band": 0,
                  "near_tie_rows": 1}
    swapped = ref["idx"].copy()
    swapped[0, 0, 0] = [0, 3, 5]               # inside the tie band
    st = bench._topk_stats(swapped, ref)
    assert st["rows_differing"] == 1 and st["rows_differing_outside_tie_band"] == 0
    wrong = ref["idx"].copy()
    wrong[0, 0, 0] = [0, 2, 6]                 # drops block 5 (above the band)
    assert bench._topk_stats(wrong, ref)["rows_differing_outside_tie_band"] == 1


def test_cold_sets():
    assert bench._cold_sets(201e6) == 4        # the dense Wan K/V
    assert bench._cold_sets(50e6) == 12        # the block-sparse path's distinct K/V
    assert bench._cold_sets(900e6) == 3
    assert bench._cold_sets(0.0) == 12


def test_counters_attach_only_to_their_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int x;  // a comment\n\nint y;\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    h = bench.src_hash([str(src)])
    (tmp_path / "profiles" / "w_counters.json").write_text(json.dumps({"code_sha256_16": h, "x": 1}))
    assert bench.counters("w", ("k.hip",))["x"] == 1
    src.write_text("int x;  // another comment\nint y;\n")      # comments and blank lines only
    assert bench.counters("w", ("k.hip",)) is not None
    src.write_text("int x;\nint z;\n")
    assert bench.counters("w", ("k.hip",)) is None
    assert bench.counters("absent", ("k.hip",)) is None

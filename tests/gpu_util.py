"""Helpers shared by the GPU parity tests: upload seeded inputs, build the ABI
shape, and compare against the oracle.  No method arithmetic lives here."""
from __future__ import annotations

import numpy as np

import dsa_inputs as g
from dsa_inputs.device import dev_to_np, shape_of, to_dev, torch, upload, upload_all  # noqa: F401

# Tolerances: per (b, t, h) row, the largest
# absolute difference over the Dc outputs must stay within RTOL * max|ref|.
RTOL = {"f32": 1e-4, "bf16": 2e-2}
# index scores are fp32 outputs: within 1e-4 of the row's largest |score|
SCORE_RTOL = 1e-4
# a selection may differ from the oracle's only by keys whose oracle scores lie
# within SWAP_GAP * max|score of the row| of the row's K-th score
SWAP_GAP = 1e-5

def assert_rows_close(got, ref, rtol, what=""):
    """got/ref [..., Dc]: per row max|got - ref| <= rtol * max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    bad = err > rtol * scale + 1e-30
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(scale, 1e-30)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} rows exceed rtol {rtol}; worst row {i}: "
                             f"err {err[i]:.3e} vs scale {scale[i]:.3e}")


def assert_scores_close(got, ref, rtol=SCORE_RTOL, what="scores"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{what}: -inf pattern differs"
    assert np.all(np.isneginf(got[~fin])), f"{what}: masked entries must be -inf"
    scale = np.where(fin, np.abs(ref), 0).max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):  # -inf - -inf on masked entries
        err = np.where(fin, np.abs(got - ref), 0)
    bad = err > rtol * scale + 1e-30
    if bad.any():
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} entries exceed rtol {rtol}; worst {i}: "
                             f"{got[i]} vs {ref[i]}")


def assert_selection_within_gap(sel_got, sel_ref, scores_ref, gap=SWAP_GAP):
    """Rows of sel_got and sel_ref (ascending, -1 padded) may differ only by
    keys whose reference scores are within gap * max|row| of the K-th score."""
    sel_got = np.asarray(sel_got)
    sel_ref = np.asarray(sel_ref)
    for r in range(sel_got.shape[0]):
        a = set(sel_got[r][sel_got[r] >= 0].tolist())
        b = set(sel_ref[r][sel_ref[r] >= 0].tolist())
        assert len(a) == len(b), f"row {r}: {len(a)} vs {len(b)} selected"
        diff = a ^ b
        if not diff:
            continue
        row = scores_ref[r].astype(np.float64)
        fin = np.isfinite(row)
        kth = row[sorted(b, key=lambda s: (-row[s], s))[-1]]
        tol = gap * np.abs(row[fin]).max()
        worst = max(abs(row[s] - kth) for s in diff)
        assert worst <= tol, f"row {r}: swapped keys {sorted(diff)[:6]} lie {worst:.3e} from the K-th score (allowed {tol:.3e})"

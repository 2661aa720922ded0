"""Helpers shared by the GPU parity tests: upload seeded inputs, build the ABI
shape, and compare against the oracle.  No method arithmetic lives here."""
from __future__ import annotations

import numpy as np

import dsa_inputs as g

# Tolerances ("Parity bar"): per (b, t, h) row, the largest
# absolute difference over the Dc outputs must stay within RTOL * max|ref|.
RTOL = {"f32": 1e-4, "bf16": 2e-2}
# index scores are fp32 outputs: within 1e-4 of the row's largest |score|
SCORE_RTOL = 1e-4
# a selection may differ from the oracle's only by keys whose oracle scores lie
# within SWAP_GAP * max|score of the row| of the row's K-th score
SWAP_GAP = 1e-5

_DT = {"f32": 0, "bf16": 1, "fp8": 2}


def torch():
    import torch as _t
    return _t


def shape_of(cfg):
    import sparse_latent_attention_lightning_amd as dsa
    return dsa.make_shape(cfg.B, cfg.T, cfg.S, cfg.HI, cfg.DI, cfg.H, cfg.Dc, cfg.Dr, cfg.K,
                          cfg.index_scale, cfg.softmax_scale, _DT[cfg.idx_dtype],
                          _DT[cfg.w_dtype], _DT[cfg.mla_dtype])


def to_dev(arr, dtype_name, device="cuda"):
    t = torch()
    arr = np.ascontiguousarray(arr)
    if dtype_name == "bf16":
        return t.from_numpy(arr.view(np.int16)).to(device).view(t.bfloat16)
    if dtype_name == "fp8":
        return t.from_numpy(arr).to(device)
    return t.from_numpy(arr.astype(np.float32)).to(device)


def upload(cfg, tensor, device="cuda"):
    """Whole ``tensor`` of ``cfg`` on the device, generated chunk by chunk.
    fp8 indexer tensors return (codes, scale bytes)."""
    t = torch()
    n = cfg.T if tensor in ("q_idx", "w", "q") else cfg.S
    tail = {"q_idx": (cfg.HI, cfg.DI), "k_idx": (cfg.DI,), "w": (cfg.HI,),
            "q": (cfg.H, cfg.D), "kv": (cfg.D,)}[tensor]
    dt = {"q_idx": cfg.idx_dtype, "k_idx": cfg.idx_dtype, "w": cfg.w_dtype,
          "q": cfg.mla_dtype, "kv": cfg.mla_dtype}[tensor]
    tdt = {"bf16": t.bfloat16, "f32": t.float32, "fp8": t.uint8}[dt]
    out = t.empty((cfg.B, n) + tail, dtype=tdt, device=device)
    sf = None
    if dt == "fp8":
        sf = t.empty((cfg.B, n) + tail[:-1] + (cfg.DI // 128,), dtype=t.uint8, device=device)
    for b, r0, r1, stored in g.iter_blocks(cfg, tensor):
        if dt == "fp8":
            out[b, r0:r1] = to_dev(stored[0], "fp8", device)
            sf[b, r0:r1] = to_dev(stored[1], "fp8", device)
        else:
            out[b, r0:r1] = to_dev(stored, dt, device)
    return (out, sf) if dt == "fp8" else out


def dev_to_np(x, dtype_name):
    t = torch()
    x = x.detach().cpu().contiguous()
    if dtype_name == "bf16":
        return x.view(t.int16).numpy().view(np.uint16)
    return x.numpy()


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

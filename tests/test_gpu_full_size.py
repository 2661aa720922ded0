"""GPU parity at each workload's full size, through dsa_forward in the launch
configuration the benchmark times (same shapes, so the same kernels, splits and
top-K plan), checked on sampled query rows the oracle computes one by one.

For each sampled row (b, t):
  * index scores from dsa_indexer_scores (the kernel dsa_forward runs) equal
    the oracle's bit for bit on integer inputs, else within 1e-4 of the row's
    largest |score|;
  * dsa_forward's selection equals the oracle's top-K of the GPU's own scores
    bit for bit, and the oracle's top-K of its own scores exactly on integer
    inputs, else up to swaps within the 1e-5 gap of the K-th score;
  * o and lse of dsa_forward match the oracle's attention over that selection
    (per (b, t, h) row within 2e-2 of max|o| for bf16).
"""
import numpy as np
import pytest

import dsa_inputs as g
import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_lightning_amd as m
    m.lib()
    oracle.build(force=False)
    return m


def _prefill_rows(cfg, extra, seed):
    fixed = [0, 1, 2046, 2047, 2048, 2049, 4095, 8191, 12287, cfg.T - 1]
    rng = np.random.default_rng(seed)
    more = rng.choice(np.setdiff1d(np.arange(cfg.T), fixed), size=extra, replace=False)
    return [(0, int(t)) for t in sorted(set(fixed) | set(more.tolist()))]


def _decode_rows(cfg, n, seed):
    if n >= cfg.B:
        return [(b, 0) for b in range(cfg.B)]
    rng = np.random.default_rng(seed)
    bs = sorted(set([0, cfg.B - 1]) | set(rng.choice(cfg.B, size=n - 2, replace=False).tolist()))
    return [(int(b), 0) for b in bs]


CASES = {
    "decode_8k": (g.CONFIGS["decode_8k"], lambda c: _decode_rows(c, 32, 11)),
    "decode_8k_int": (g.CONFIGS["decode_8k"].replace(integer=True), lambda c: _decode_rows(c, 8, 12)),
    "prefill_16k": (g.CONFIGS["prefill_16k"], lambda c: _prefill_rows(c, 6, 13)),
    "decode_128k": (g.CONFIGS["decode_128k"], lambda c: _decode_rows(c, 8, 14)),
    "decode_64k_fp8": (g.CONFIGS["decode_64k_fp8"], lambda c: _decode_rows(c, 6, 15)),
    "decode_64k_fp8_int": (g.CONFIGS["decode_64k_fp8"].replace(integer=True), lambda c: _decode_rows(c, 4, 16)),
    "prefill_16k_fp8": (g.CONFIGS["prefill_16k_fp8"], lambda c: _prefill_rows(c, 4, 17)),
}


def _inputs(cfg):
    d = {n: U.upload(cfg, n) for n in ("q_idx", "k_idx", "w", "q", "kv")}
    if cfg.idx_dtype == "fp8":
        d["q_idx"], d["q_sf"] = d["q_idx"]
        d["k_idx"], d["k_sf"] = d["k_idx"]
    else:
        d["q_sf"] = d["k_sf"] = None
    return d


def _per_query(cfg, tensor, picks):
    parts = [g.rows(cfg, tensor, b, t, t + 1) for b, t in picks]
    if isinstance(parts[0], tuple):
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    return np.concatenate(parts)


def _per_sequence(cfg, tensor, seqs):
    parts = [g.rows(cfg, tensor, b, 0, cfg.S) for b in seqs]
    if isinstance(parts[0], tuple):
        return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])
    return np.stack(parts)


@pytest.mark.parametrize("case", list(CASES))
def test_full_size_forward(dsa, case):
    torch = U.torch()
    cfg, pick_rows = CASES[case]
    picks = pick_rows(cfg)
    print(f"[full-size] {case}: {cfg}; {len(picks)} sampled rows", flush=True)
    x = _inputs(cfg)
    shape = U.shape_of(cfg)
    o, lse, idx = dsa.dsa_forward(shape, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                  x["q_sf"], x["k_sf"])
    scores = dsa.dsa_indexer_scores(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"])
    torch.cuda.synchronize()
    del x
    flat = [b * cfg.T + t for b, t in picks]
    sel = torch.tensor(flat, dtype=torch.int64, device="cuda")
    got_sc = scores.view(cfg.B * cfg.T, cfg.S).index_select(0, sel).cpu().numpy()
    got_idx = idx.view(cfg.B * cfg.T, -1).index_select(0, sel).cpu().numpy()
    got_o = U.dev_to_np(o.view(cfg.B * cfg.T, cfg.H, cfg.Dc).index_select(0, sel), "bf16")
    got_o = g.bf16_bits_to_f32(got_o)
    got_lse = lse.view(cfg.B * cfg.T, cfg.H).index_select(0, sel).cpu().numpy()
    del o, lse, idx, scores
    torch.cuda.empty_cache()

    # the oracle sees only the sequences the sampled rows belong to
    seqs = sorted(set(b for b, _ in picks))
    sub = cfg.replace(B=len(seqs))
    rb = np.array([seqs.index(b) for b, _ in picks], np.int32)
    rt = np.array([t for _, t in picks], np.int32)
    qi = _per_query(cfg, "q_idx", picks)
    w = _per_query(cfg, "w", picks)
    k = _per_sequence(cfg, "k_idx", seqs)
    if cfg.idx_dtype == "fp8":
        ref_sc = oracle.indexer_scores(sub, rb, rt, qi[0], w, k[0], qi[1], k[1])
    else:
        ref_sc = oracle.indexer_scores(sub, rb, rt, qi, w, k)
    del k
    if cfg.integer:
        assert np.array_equal(got_sc, ref_sc), f"{case}: integer scores must be bit-exact"
    else:
        U.assert_scores_close(got_sc, ref_sc, what=f"{case} scores")

    # selection: exact on the GPU's own scores; against the oracle's scores,
    # exact on integers, else within the swap gap
    assert np.array_equal(got_idx, oracle.topk(sub, got_sc)), f"{case}: top-K of the GPU scores differs"
    ref_idx = oracle.topk(sub, ref_sc)
    if cfg.integer:
        assert np.array_equal(got_idx, ref_idx), f"{case}: selection must be bit-exact"
    else:
        U.assert_selection_within_gap(got_idx, ref_idx, ref_sc)

    q = _per_query(cfg, "q", picks).reshape(len(picks), cfg.H, cfg.D)
    kv = _per_sequence(cfg, "kv", seqs)
    ro, rl = oracle.sparse_mla(sub, rb, q, kv, got_idx)
    U.assert_rows_close(got_o, ro, U.RTOL["bf16"], what=f"{case} o")
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(got_lse))
    assert np.all(np.abs(got_lse[fin] - rl[fin]) <= U.RTOL["bf16"] * np.maximum(1, np.abs(rl[fin])))
    if case == "decode_128k":
        # the planted cluster: report how much of the selection falls inside it
        inside = [np.isin(got_idx[i], g.cluster_positions(cfg, seqs[rb[i]])).mean() for i in range(len(picks))]
        print(f"[full-size] decode_128k: {np.mean(inside):.1%} of the selected keys are cluster keys", flush=True)

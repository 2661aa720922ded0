"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle routine to a hand-worked example, a closed form, an
invariant, or a special case that reduces to a library routine (numpy matmul,
numpy lexsort, torch's scaled_dot_product_attention in fp64).  The shapes are
deliberately non-square (HI != DI, T != S, Dc != Dr) so that a transposed
operand or a swapped index changes the result.
"""
import json
import math
import os

import numpy as np
import pytest

import dsa_inputs as g
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(**kw):
    base = dict(name="pin", B=2, T=5, S=37, HI=3, DI=7, H=3, Dc=6, Dr=2, K=8,
                idx_dtype="f32", w_dtype="f32", mla_dtype="f32", seed=11)
    base.update(kw)
    return g.Config(**base)


def _rows(cfg):
    rb = np.repeat(np.arange(cfg.B, dtype=np.int32), cfg.T)
    rt = np.tile(np.arange(cfg.T, dtype=np.int32), cfg.B)
    return rb, rt


def _draw(cfg, rng, integer=False):
    def d(*shape):
        if integer:
            return rng.integers(-3, 4, size=shape).astype(np.float32)
        return rng.standard_normal(shape).astype(np.float32)
    return dict(q_idx=d(cfg.B * cfg.T, cfg.HI, cfg.DI), k_idx=d(cfg.B, cfg.S, cfg.DI),
                w=d(cfg.B * cfg.T, cfg.HI), q=d(cfg.B * cfg.T, cfg.H, cfg.D),
                kv=d(cfg.B, cfg.S, cfg.D))


def _scores(cfg, x):
    rb, rt = _rows(cfg)
    return oracle.indexer_scores(cfg, rb, rt, x["q_idx"], x["w"], x["k_idx"])


def _causal_mask(cfg):
    rb, rt = _rows(cfg)
    qpos = cfg.S - cfg.T + rt
    return np.arange(cfg.S)[None, :] <= qpos[:, None]


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def _num(v):
    if v == "-inf":
        return -math.inf
    if v == "ln3":
        return math.log(3.0)
    if v == "ln4":
        return math.log(4.0)
    return float(v)


def test_worked_example_indexer(oracle_lib):
    ex = _golden()["indexer"]
    q = np.array(ex["q_idx"], np.float32)[None]
    k = np.array(ex["k_idx"], np.float32)[None]
    w = np.array(ex["w"], np.float32)[None]
    dec = _cfg(B=1, T=1, S=3, HI=2, DI=2, K=2, idx_scale=ex["idx_scale"])
    s = oracle.indexer_scores(dec, [0], [0], q, w, k)
    assert s[0].tolist() == [_num(v) for v in ex["decode_scores"]]
    assert oracle.topk(dec, s)[0].tolist() == ex["decode_topk"]
    pre = dec.replace(T=3)
    s = oracle.indexer_scores(pre, [0], [0], q, w, k)
    assert s[0].tolist() == [_num(v) for v in ex["prefill_t0_scores"]]
    assert oracle.topk(pre, s)[0].tolist() == ex["prefill_t0_topk"]


def test_worked_example_attention(oracle_lib):
    ex = _golden()["attention"]
    cfg = _cfg(B=1, T=1, S=3, H=1, Dc=2, Dr=1, sm_scale=ex["sm_scale"])
    kv = np.array(ex["kv"], np.float64)[None].astype(np.float32)
    q = np.array([[[_num(v) for v in ex["q"]]]], np.float32)
    idx = np.array([ex["idx"]], np.int32)
    o, lse, p = oracle.sparse_mla(cfg, [0], q, kv, idx, want_probs=True)
    np.testing.assert_allclose(o[0, 0], ex["o"], rtol=1e-6)
    np.testing.assert_allclose(p[0, 0], ex["probs"], rtol=1e-6, atol=1e-12)
    assert abs(lse[0, 0] - _num(ex["lse"])) < 1e-6


# ---------------------------------------------------------------------------
# index scores
# ---------------------------------------------------------------------------

def test_scores_single_head_unit_weight_is_relu_matmul(oracle_lib):
    """HI = 1, w = 1: S = scale * ReLU(Q K^T) (numpy matmul), exact on integers."""
    cfg = _cfg(HI=1)
    rng = np.random.default_rng(1)
    x = _draw(cfg, rng, integer=True)
    x["w"][:] = 1.0
    s = _scores(cfg, x)
    rb, _ = _rows(cfg)
    ref = np.einsum("nd,nsd->ns", x["q_idx"][:, 0].astype(np.int64),
                    x["k_idx"][rb].astype(np.int64))
    ref = np.float32(cfg.index_scale) * np.maximum(ref, 0).astype(np.float32)
    mask = _causal_mask(cfg)
    assert np.array_equal(s[mask], ref[mask])
    assert np.all(np.isneginf(s[~mask]))


def test_scores_relu_sits_between_dot_and_weight(oracle_lib):
    """Heads (q, -q) with w = (1, -1) give scale*(q.k); with w = (1, 1), scale*|q.k|.

    relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x|: a missing ReLU, a
    ReLU after the weight, or a dropped head changes one of the two."""
    cfg = _cfg(HI=2, T=1)
    rng = np.random.default_rng(2)
    x = _draw(cfg, rng, integer=True)
    x["q_idx"][:, 1] = -x["q_idx"][:, 0]
    rb, _ = _rows(cfg)
    dot = np.einsum("nd,nsd->ns", x["q_idx"][:, 0], x["k_idx"][rb]).astype(np.float32)
    sc = np.float32(cfg.index_scale)
    x["w"][:] = [1.0, -1.0]
    assert np.array_equal(_scores(cfg, x), sc * dot)
    x["w"][:] = [1.0, 1.0]
    assert np.array_equal(_scores(cfg, x), sc * np.abs(dot))


def test_scores_nonnegative_dots_are_linear_in_weighted_query(oracle_lib):
    """All q.k >= 0: S = scale * ((sum_h w_h q_h) . k), a plain GEMV."""
    cfg = _cfg(T=2)
    rng = np.random.default_rng(3)
    x = _draw(cfg, rng)
    x["q_idx"] = np.abs(x["q_idx"])
    x["k_idx"] = np.abs(x["k_idx"])
    s = _scores(cfg, x).astype(np.float64)
    rb, _ = _rows(cfg)
    u = np.einsum("nh,nhd->nd", x["w"].astype(np.float64), x["q_idx"].astype(np.float64))
    ref = cfg.index_scale * np.einsum("nd,nsd->ns", u, x["k_idx"][rb].astype(np.float64))
    mask = _causal_mask(cfg)
    np.testing.assert_allclose(s[mask], ref[mask], rtol=2e-6, atol=1e-6)


def test_scores_causal_boundary_and_decode_alignment(oracle_lib):
    """Query t sits at S - T + t and sees keys 0..S-T+t (diagonal included)."""
    rng = np.random.default_rng(4)
    for T, S in [(5, 37), (1, 9), (9, 9)]:
        cfg = _cfg(T=T, S=S)
        x = _draw(cfg, rng)
        x["q_idx"] = np.abs(x["q_idx"])
        x["k_idx"] = np.abs(x["k_idx"]) + 0.5
        x["w"] = np.abs(x["w"]) + 0.5
        s = _scores(cfg, x)
        _, rt = _rows(cfg)
        finite = np.isfinite(s).sum(axis=1)
        assert np.array_equal(finite, S - T + rt + 1)
        assert np.all(s[np.isfinite(s)] > 0)


def test_scores_ragged_lengths(oracle_lib):
    """Per-sequence context lengths L_b: sequence b's queries sit at
    L_b - T + t and see keys 0 .. L_b - T + t, never one at or past L_b; a
    query whose position is negative sees nothing.  Checked against the int64
    closed form on integer inputs (lengths S, inside, equal to T, below T, 0)."""
    lens = [37, 20, 5, 3, 0]
    cfg = _cfg(B=len(lens))
    rng = np.random.default_rng(12)
    x = _draw(cfg, rng, integer=True)
    rb, rt = _rows(cfg)
    s = oracle.indexer_scores(cfg, rb, rt, x["q_idx"], x["w"], x["k_idx"],
                              seq_lens=np.array(lens, np.int32))
    d = np.einsum("nhd,nsd->nhs", x["q_idx"].astype(np.int64),
                  x["k_idx"][rb].astype(np.int64))
    acc = np.einsum("nh,nhs->ns", x["w"].astype(np.int64), np.maximum(d, 0))
    ref = np.float32(cfg.index_scale) * acc.astype(np.float32)
    qpos = np.array(lens, np.int64)[rb] - cfg.T + rt
    vis = np.arange(cfg.S)[None, :] <= qpos[:, None]
    assert np.array_equal(np.isfinite(s), vis)
    assert np.array_equal(s[vis], ref[vis])
    assert np.all(s[~vis] == -np.inf)
    # lengths of S everywhere are the unragged call
    full = oracle.indexer_scores(cfg, rb, rt, x["q_idx"], x["w"], x["k_idx"],
                                 seq_lens=np.full(cfg.B, cfg.S, np.int32))
    assert np.array_equal(full, _scores(cfg, x))


def test_scores_integer_mode_exact_against_int64(oracle_lib):
    """Integer inputs in [-3, 3]: the score equals the int64 closed form, scaled."""
    cfg = g.CONFIGS["tiny"]
    qi = g.full(cfg, "q_idx")[0]
    ki = g.full(cfg, "k_idx")
    w = g.full(cfg, "w")[0]
    rb = np.zeros(cfg.T, np.int32)
    rt = np.arange(cfg.T, dtype=np.int32)
    s = oracle.indexer_scores(cfg, rb, rt, qi, w, ki)
    d = np.einsum("thd,sd->ths", qi.astype(np.int64), ki[0].astype(np.int64))
    acc = np.einsum("th,ths->ts", w.astype(np.int64), np.maximum(d, 0))
    ref = np.float32(cfg.index_scale) * acc.astype(np.float32)
    mask = np.tril(np.ones((cfg.T, cfg.S), bool))
    assert np.array_equal(s[mask], ref[mask])


def test_scores_bf16_inputs_are_read_exactly(oracle_lib):
    """bf16 storage decodes exactly: same scores as the fp32 copy of the values."""
    cfg = _cfg(T=2)
    rng = np.random.default_rng(5)
    x = _draw(cfg, rng)
    xb = {k: g.f32_to_bf16_bits(v) for k, v in x.items()}
    xf = {k: g.bf16_bits_to_f32(v) for k, v in xb.items()}
    s_b = _scores(cfg.replace(idx_dtype="bf16", w_dtype="bf16"), xb)
    s_f = _scores(cfg, xf)
    assert np.array_equal(s_b, s_f)


def test_scores_fp8_block_scales(oracle_lib):
    """e4m3 with ue8m0 scales: byte 127 reproduces the integer result exactly;
    raising the query scale byte by a and the key byte by b multiplies every
    score by 2^(a+b) exactly (two blocks per row: DI = 256)."""
    cfg = _cfg(DI=256, T=2, idx_dtype="fp8")
    rng = np.random.default_rng(6)
    x = _draw(cfg, rng, integer=True)
    qc, kc = g.f32_to_e4m3(x["q_idx"]), g.f32_to_e4m3(x["k_idx"])
    qs = np.full(x["q_idx"].shape[:-1] + (2,), 127, np.uint8)
    ks = np.full(x["k_idx"].shape[:-1] + (2,), 127, np.uint8)
    rb, rt = _rows(cfg)
    s8 = oracle.indexer_scores(cfg, rb, rt, qc, x["w"], kc, qs, ks)
    s32 = _scores(cfg.replace(idx_dtype="f32"), x)
    assert np.array_equal(s8, s32)
    s8b = oracle.indexer_scores(cfg, rb, rt, qc, x["w"], kc, qs + 2, ks - 5)
    mask = np.isfinite(s32)
    assert np.array_equal(s8b[mask], s32[mask] * np.float32(2.0 ** -3))
    # one block scaled on its own only scales that block's contribution
    x2 = dict(x)
    x2["q_idx"] = x["q_idx"].copy()
    x2["q_idx"][..., 128:] *= 4.0
    qs2 = qs.copy()
    qs2[..., 1] += 2
    s8c = oracle.indexer_scores(cfg, rb, rt, qc, x["w"], kc, qs2, ks)
    s32c = _scores(cfg.replace(idx_dtype="f32"), x2)
    assert np.array_equal(s8c, s32c)


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------

def _lexsort_topk(row, K):
    """Reference selection with numpy.lexsort on (score desc, index asc)."""
    idx = np.arange(row.size)
    ok = ~(np.isnan(row) | np.isneginf(row))
    r, i = row[ok].astype(np.float64), idx[ok]
    r = np.where(r == 0.0, 0.0, r)  # -0 == +0
    order = np.lexsort((i, -r))
    sel = np.sort(i[order[:K]])
    out = -np.ones(min(K, row.size), np.int64)
    out[: sel.size] = sel
    return out


def test_topk_matches_lexsort_with_heavy_ties(oracle_lib):
    rng = np.random.default_rng(7)
    for S, K in [(37, 8), (64, 64), (100, 130), (257, 31)]:
        cfg = _cfg(S=S, K=K, T=1)
        sc = rng.integers(-4, 5, size=(20, S)).astype(np.float32)
        sc[3] = 0.0
        sc[4, ::3] = -0.0
        sc[5, ::2] = -np.inf
        sc[6, 1::4] = np.nan
        sc[7] = -np.inf
        sc[8, 5] = np.inf
        got = oracle.topk(cfg, sc)
        for r in range(sc.shape[0]):
            assert np.array_equal(got[r], _lexsort_topk(sc[r], K)), (S, K, r)


def test_topk_invariants_real_scores(oracle_lib):
    """Every selected score >= every unselected one; equal scores at the
    boundary go to the lower indices; output ascending then -1."""
    rng = np.random.default_rng(8)
    cfg = _cfg(S=500, K=64, T=1)
    sc = rng.standard_normal((16, 500)).astype(np.float32)
    sc[:, 300:310] = sc[:, 10:11]  # a block of equal values
    got = oracle.topk(cfg, sc)
    for r in range(16):
        sel = got[r][got[r] >= 0]
        assert np.all(np.diff(sel) > 0)
        mask = np.zeros(500, bool)
        mask[sel] = True
        assert sel.size == 64
        lo = sc[r][mask].min()
        assert sc[r][~mask].max() <= lo
        eq_sel = np.nonzero(mask & (sc[r] == lo))[0]
        eq_uns = np.nonzero(~mask & (sc[r] == lo))[0]
        if eq_uns.size:
            assert eq_sel.max() < eq_uns.min()


def test_topk_signed_zero_is_one_value(oracle_lib):
    cfg = _cfg(S=6, K=3, T=1)
    sc = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0, 1.0]], np.float32)
    assert oracle.topk(cfg, sc)[0].tolist() == [0, 1, 5]


def test_topk_short_rows_pad_and_wide_k(oracle_lib):
    cfg = _cfg(S=6, K=10, T=1)
    sc = np.array([[1, -np.inf, 2, np.nan, -np.inf, 0]], np.float32)
    assert oracle.topk(cfg, sc)[0].tolist() == [0, 2, 5, -1, -1, -1]


# ---------------------------------------------------------------------------
# latent attention
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, mask=None):
    """torch scaled_dot_product_attention in fp64 on the CPU, [H, Tq, D]."""
    torch = pytest.importorskip("torch")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a, np.float64)) for a in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=1.0)
    return out.numpy()


def test_sparse_with_full_selection_is_dense_causal_sdpa(oracle_lib):
    """K >= causal length: top-k keeps every visible key, and sparse attention
    equals textbook causal softmax attention (torch SDPA, fp64) to 1e-12;
    row t has exactly t + 1 nonzero probabilities."""
    cfg = _cfg(B=1, T=24, S=24, K=24, H=3, Dc=6, Dr=2, sm_scale=0.37)
    rng = np.random.default_rng(9)
    x = _draw(cfg, rng)
    rb, rt = _rows(cfg)
    idx = oracle.topk(cfg, _scores(cfg, x))
    o, lse, p = oracle.sparse_mla(cfg, rb, x["q"], x["kv"], idx, want_probs=True)
    kv = x["kv"][0].astype(np.float64)
    sm = np.float64(np.float32(cfg.sm_scale))                            # the scale is an fp32 argument
    q = x["q"].astype(np.float64).transpose(1, 0, 2) * sm                # [H, T, D]
    k = np.broadcast_to(kv[None], (cfg.H,) + kv.shape)                   # one key row for all heads
    v = np.broadcast_to(kv[None, :, : cfg.Dc], (cfg.H, cfg.S, cfg.Dc))   # value = latent part
    ref = _sdpa(q, k, v, mask=np.tril(np.ones((cfg.T, cfg.S), bool)))
    np.testing.assert_allclose(o.transpose(1, 0, 2), ref, rtol=1e-12, atol=1e-12)
    nz = (p[:, 0, :] != 0).sum(axis=1)
    assert np.array_equal(nz, np.arange(1, cfg.T + 1))
    do, dl = oracle.dense_mla(cfg, rb, rt, x["q"], x["kv"])
    np.testing.assert_allclose(o, do, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, dl, rtol=1e-12, atol=1e-12)


def test_absorbed_equals_explicit_form(oracle_lib):
    """q_lat_h = W_UK,h q^C_h and out_h = o_lat_h W_UV,h reproduce the explicit
    per-head keys c W_UK and values c W_UV, checked against both the oracle's
    explicit routine and torch SDPA on explicitly expanded keys (fp64, 1e-12)."""
    rng = np.random.default_rng(10)
    H, Dc, Dn, Dv, Dr, S = 4, 16, 8, 6, 4, 13
    sm = 0.29
    qC = rng.standard_normal((H, Dn))
    qR = rng.standard_normal((H, Dr))
    kv = rng.standard_normal((S, Dc + Dr))
    c, r = kv[:, :Dc], kv[:, Dc:]
    W_UK = rng.standard_normal((Dc, H * Dn)) / 4
    W_UV = rng.standard_normal((Dc, H * Dv)) / 4
    explicit = oracle.explicit_mla(qC, qR, c, r, W_UK, W_UV, sm)
    # library form: expand keys and values per head, then SDPA
    KC = (c @ W_UK).reshape(S, H, Dn).transpose(1, 0, 2)
    Kfull = np.concatenate([KC, np.broadcast_to(r[None], (H, S, Dr))], axis=-1)
    V = (c @ W_UV).reshape(S, H, Dv).transpose(1, 0, 2)
    qfull = np.concatenate([qC, qR], axis=-1)[:, None, :] * sm
    ref = _sdpa(qfull, Kfull, V)[:, 0]
    np.testing.assert_allclose(explicit, ref, rtol=1e-12, atol=1e-12)
    # absorbed form through the sparse routine
    q_lat = np.stack([W_UK[:, h * Dn:(h + 1) * Dn] @ qC[h] for h in range(H)])
    q_abs = np.concatenate([q_lat, qR], axis=-1)[None].astype(np.float64)
    cfg = _cfg(B=1, T=1, S=S, H=H, Dc=Dc, Dr=Dr, K=S, sm_scale=sm)
    # the oracle reads fp32 storage: keep values exactly representable
    q32 = q_abs.astype(np.float32)
    kv32 = kv[None].astype(np.float32)
    o_lat, _ = oracle.sparse_mla(cfg, [0], q32, kv32, np.arange(S, dtype=np.int32)[None])
    out = np.stack([o_lat[0, h] @ W_UV[:, h * Dv:(h + 1) * Dv] for h in range(H)])
    # same identity on the rounded inputs, through torch, to 1e-12
    c32, r32 = kv32[0, :, :Dc].astype(np.float64), kv32[0, :, Dc:].astype(np.float64)
    qa = q32[0].astype(np.float64)
    ref_abs = _sdpa(qa[:, None, :] * np.float64(np.float32(sm)),
                    np.broadcast_to(np.concatenate([c32, r32], 1)[None], (H, S, Dc + Dr)),
                    np.broadcast_to(c32[None], (H, S, Dc)))[:, 0]
    np.testing.assert_allclose(o_lat[0], ref_abs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, ref, rtol=2e-5, atol=2e-5)  # fp32 rounding of q, kv


def test_softmax_rows_sum_to_one(oracle_lib):
    cfg = _cfg(B=2, T=3, S=50, K=16)
    rng = np.random.default_rng(12)
    x = _draw(cfg, rng)
    rb, _ = _rows(cfg)
    idx = oracle.topk(cfg, _scores(cfg, x))
    _, _, p = oracle.sparse_mla(cfg, rb, x["q"], x["kv"], idx, want_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[np.broadcast_to((idx < 0)[:, None, :], p.shape)] == 0)


def test_zero_query_averages_selected_latents(oracle_lib):
    """q = 0: every logit is 0, o = mean of the selected latent rows, lse = ln |J|."""
    cfg = _cfg(B=1, T=1, S=40, K=9)
    rng = np.random.default_rng(13)
    kv = rng.standard_normal((1, 40, cfg.D)).astype(np.float32)
    q = np.zeros((1, cfg.H, cfg.D), np.float32)
    idx = np.array([[3, 7, 8, 11, 20, 21, 39, -1, -1]], np.int32)
    o, lse = oracle.sparse_mla(cfg, [0], q, kv, idx)
    ref = kv[0, idx[0][idx[0] >= 0], : cfg.Dc].astype(np.float64).mean(0)
    for h in range(cfg.H):
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(7), rtol=1e-14)


def test_single_key_and_duplicates_and_empty_rows(oracle_lib):
    cfg = _cfg(B=1, T=1, S=10, K=4, sm_scale=0.5)
    rng = np.random.default_rng(14)
    kv = rng.standard_normal((1, 10, cfg.D)).astype(np.float32)
    q = rng.standard_normal((1, cfg.H, cfg.D)).astype(np.float32)
    logit = 0.5 * (q[0].astype(np.float64) @ kv[0, 6].astype(np.float64))
    o, lse = oracle.sparse_mla(cfg, [0], q, kv, np.array([[6, -1, 55, -7]], np.int32))
    np.testing.assert_allclose(o[0], np.broadcast_to(kv[0, 6, : cfg.Dc], (cfg.H, cfg.Dc)),
                               rtol=1e-14)
    np.testing.assert_allclose(lse[0], logit, rtol=1e-12)
    # a duplicate counts twice: same output, lse + ln 2
    o2, lse2 = oracle.sparse_mla(cfg, [0], q, kv, np.array([[6, 6, -1, -1]], np.int32))
    np.testing.assert_allclose(o2, o, rtol=1e-14)
    np.testing.assert_allclose(lse2[0], logit + math.log(2), rtol=1e-12)
    o3, lse3 = oracle.sparse_mla(cfg, [0], q, kv, np.array([[-1, -1, 10, -2]], np.int32))
    assert np.all(o3 == 0) and np.all(np.isneginf(lse3))


def test_index_order_does_not_matter(oracle_lib):
    cfg = _cfg(B=1, T=1, S=64, K=12)
    rng = np.random.default_rng(15)
    kv = rng.standard_normal((1, 64, cfg.D)).astype(np.float32)
    q = rng.standard_normal((1, cfg.H, cfg.D)).astype(np.float32)
    idx = np.sort(rng.choice(64, 12, replace=False)).astype(np.int32)[None]
    o1, l1 = oracle.sparse_mla(cfg, [0], q, kv, idx)
    o2, l2 = oracle.sparse_mla(cfg, [0], q, kv, idx[:, ::-1].copy())
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_rotary_part_enters_logits_not_values(oracle_lib):
    """Zeroing q's latent part leaves logits from the rotary part only; the
    output is still a mix of the latent columns (never the rotary ones)."""
    cfg = _cfg(B=1, T=1, S=5, K=5, H=1, Dc=3, Dr=2, sm_scale=1.0)
    kv = np.zeros((1, 5, 5), np.float32)
    kv[0, :, :3] = np.arange(15, dtype=np.float32).reshape(5, 3)
    kv[0, 2, 3:] = [1.0, 1.0]
    q = np.array([[[0, 0, 0, 20.0, 20.0]]], np.float32)
    o, lse = oracle.sparse_mla(cfg, [0], q, kv, np.arange(5, dtype=np.int32)[None])
    np.testing.assert_allclose(o[0, 0], kv[0, 2, :3], rtol=1e-12)  # weight ~ 1 on key 2
    np.testing.assert_allclose(lse[0, 0], 40.0, rtol=1e-12)


# ---------------------------------------------------------------------------
# page constants
# ---------------------------------------------------------------------------

def test_page_constants_fix_the_shapes():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        pc = json.load(f)
    v = {k: (d["value"] if isinstance(d, dict) else d) for k, d in pc.items() if not k.startswith("_")}
    dim, qr, kr = v["dim"], v["q_lora_rank"], v["kv_lora_rank"]
    H, dn, dr, dv = v["n_heads"], v["qk_nope_head_dim"], v["qk_rope_head_dim"], v["v_head_dim"]
    HI, DI = v["index_n_heads"], v["index_head_dim"]
    params = (dim * qr + qr + qr * H * (dn + dr) + dim * (kr + dr) + kr + kr * H * (dn + dv)
              + H * dv * dim
              + qr * HI * DI + dim * DI + 2 * DI + dim * HI)   # indexer: wq_b, wk, LayerNorm(w, b), weights_proj
    assert params == v["sparse_latent_attention_params_per_block"]
    # the shapes the workloads use
    for name in ("decode_8k", "prefill_16k", "decode_128k", "decode_64k_fp8"):
        c = g.CONFIGS[name]
        assert (c.HI, c.DI, c.H, c.Dc, c.Dr, c.K) == (HI, DI, H, kr, dr, v["index_topk"])
        assert abs(c.softmax_scale - (dn + dr) ** -0.5) < 1e-7
        assert abs(c.index_scale - 1 / (math.sqrt(HI) * math.sqrt(DI))) < 1e-9
    assert round((dn + dr) ** -0.5, 4) == v["softmax_scale_plain"]
    for ver in ("v32", "v2"):
        f = v[f"yarn_factor_{ver}"]
        d = pc[f"yarn_factor_{ver}"]
        m = (0.1 * d["mscale"] * math.log(d["rope_factor"]) + 1.0) ** 2
        assert round(m, 2) == f
        assert round(m * (dn + dr) ** -0.5, 4) == v[f"softmax_scale_yarn_{ver}"]


# ---------------------------------------------------------------------------
# cache fill and indexer inputs (the step before the path)
# ---------------------------------------------------------------------------

def _fill_inputs(n=4, D=96, seed=21):
    rng = np.random.default_rng(seed)
    x = g.f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32))
    W = g.f32_to_bf16_bits((rng.standard_normal((oracle.FILL_COLS, D)) / 8).astype(np.float32))
    ang = rng.uniform(-math.pi, math.pi, (n, 32))
    return x, W, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _proj(x, W):
    """The joint projection by numpy's matmul on the exact bf16 values."""
    return g.bf16_bits_to_f32(x).astype(np.float64) @ g.bf16_bits_to_f32(W).astype(np.float64).T


def test_fill_projection_is_the_matmul(oracle_lib):
    """w is the raw projection; the other three blocks are functions of theirs."""
    x, W, c, s = _fill_inputs()
    _, _, w = oracle.cache_fill(x, W, np.ones(512), np.ones(128), np.zeros(128), c, s)
    np.testing.assert_allclose(w, _proj(x, W)[:, 704:768], rtol=1e-12, atol=1e-12)


def test_fill_latent_rmsnorm(oracle_lib):
    """gain 1: unit root-mean-square; scale invariant (x doubled, exact in
    bf16); the gain multiplies elementwise."""
    x, W, c, s = _fill_inputs()
    ones, zeros = np.ones(128), np.zeros(128)
    kv, _, _ = oracle.cache_fill(x, W, np.ones(512), ones, zeros, c, s)
    rms = np.sqrt((kv[:, :512] ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1) < 1e-5)
    x2 = g.f32_to_bf16_bits(2 * g.bf16_bits_to_f32(x))
    kv2, _, _ = oracle.cache_fill(x2, W, np.ones(512), ones, zeros, c, s)
    np.testing.assert_allclose(kv2[:, :512], kv[:, :512], rtol=1e-5, atol=1e-6)
    gain = np.linspace(-2, 3, 512).astype(np.float32)
    kvg, _, _ = oracle.cache_fill(x, W, gain, ones, zeros, c, s)
    np.testing.assert_allclose(kvg[:, :512], kv[:, :512] * gain, rtol=1e-12, atol=1e-12)
    # direction: the normalised latent is parallel to the raw one
    raw = _proj(x, W)[:, :512]
    cos = (kv[:, :512] * raw).sum(1) / np.linalg.norm(kv[:, :512], axis=1) / np.linalg.norm(raw, axis=1)
    assert np.all(cos > 1 - 1e-12)


def test_fill_rotary_layout_and_rotation(oracle_lib):
    """Angle 0: the rotary part is the projection's even dims, then its odd
    ones (the nnterp deepseek_v32 page, section 02); a quarter turn maps
    (a, b) to (-b, a); every rotation keeps each pair's length."""
    x, W, c, s = _fill_inputs()
    n = x.shape[0]
    ones, zeros = np.ones(128), np.zeros(128)
    kpe = _proj(x, W)[:, 512:576]
    kv, _, _ = oracle.cache_fill(x, W, np.ones(512), ones, zeros, np.ones((n, 32)), np.zeros((n, 32)))
    np.testing.assert_allclose(kv[:, 512:544], kpe[:, 0::2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kv[:, 544:576], kpe[:, 1::2], rtol=1e-12, atol=1e-12)
    kv, _, _ = oracle.cache_fill(x, W, np.ones(512), ones, zeros, np.zeros((n, 32)), np.ones((n, 32)))
    np.testing.assert_allclose(kv[:, 512:544], -kpe[:, 1::2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kv[:, 544:576], kpe[:, 0::2], rtol=1e-12, atol=1e-12)
    kv, _, _ = oracle.cache_fill(x, W, np.ones(512), ones, zeros, c, s)
    np.testing.assert_allclose(kv[:, 512:544] ** 2 + kv[:, 544:576] ** 2,
                               kpe[:, 0::2] ** 2 + kpe[:, 1::2] ** 2, rtol=1e-6)


def test_fill_indexer_key_layernorm(oracle_lib):
    """gain 1, bias 0: zero mean and unit variance; gain and bias are affine."""
    x, W, c, s = _fill_inputs()
    _, k, _ = oracle.cache_fill(x, W, np.ones(512), np.ones(128), np.zeros(128), c, s)
    assert np.all(np.abs(k.mean(axis=1)) < 1e-12)
    assert np.all(np.abs(k.var(axis=1) - 1) < 1e-5)
    gam = np.linspace(0.5, 2, 128).astype(np.float32)
    bet = np.linspace(-1, 1, 128).astype(np.float32)
    _, k2, _ = oracle.cache_fill(x, W, np.ones(512), gam, bet, c, s)
    np.testing.assert_allclose(k2, k * gam + bet, rtol=1e-12, atol=1e-12)
    # the raw projection's own centring and scale
    raw = _proj(x, W)[:, 576:704]
    z = (raw - raw.mean(1, keepdims=True)) / np.sqrt(raw.var(1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(k, z, rtol=1e-9, atol=1e-9)


def test_quantize_e4m3_blocks(oracle_lib):
    """The block quantiser against the input generator's numpy version, and
    hand-worked cases: exact codes, ties to even, scale at and above a power of
    two, the all-zero block, the subnormal range."""
    rng = np.random.default_rng(22)
    y = rng.standard_normal((6, 256)) * np.array([1e-3, 1, 7, 300, 2e4, 0.02])[:, None]
    y[2, :128] = 0.0
    codes, sb = oracle.quantize_e4m3(y)
    c2, s2 = g.quantize_e4m3_blocks(y.astype(np.float32))
    assert np.array_equal(codes, c2) and np.array_equal(sb, s2)
    blk = np.zeros(128)
    blk[:6] = [448.0, 1.0625, 1.1875, -2.5, 2.0 ** -9 * 1.5, 2.0 ** -9 * 0.5]
    codes, sb = oracle.quantize_e4m3(blk)
    assert sb.tolist() == [127]                               # 448 fits exactly: scale 1
    assert codes[:6].tolist() == [0x7E, 0x38, 0x3A, 0xC2, 0x02, 0x00]
    blk[0] = 448.0 * 1.0001                                   # just above: next power of two
    _, sb = oracle.quantize_e4m3(blk)
    assert sb.tolist() == [128]
    _, sb = oracle.quantize_e4m3(np.zeros(128))
    assert sb.tolist() == [127]
    # the scale byte holds 2^(byte - 127) for bytes 0..254: a block whose
    # largest magnitude lies below 448 2^-127 keeps the smallest scale, byte 0
    # (the exponent would otherwise wrap the byte), and its codes stay finite
    for amax in (1e-37, 3e-39, 1e-45, 448.0 * 2.0 ** -127):
        blk = np.zeros(128)
        blk[3] = -amax
        blk[9] = amax / 3
        codes, sb = oracle.quantize_e4m3(blk)
        assert sb.tolist() == [0], (amax, sb)
        c2, s2 = g.quantize_e4m3_blocks(blk.astype(np.float32))
        assert np.array_equal(sb, s2) and np.array_equal(codes, c2)
        assert codes[3] & 0x80 and (codes[3] & 0x7F) <= 0x7E
    blk = np.zeros(128)
    blk[0] = 448.0 * 2.0 ** -126                              # the largest scale-byte-1 block
    _, sb = oracle.quantize_e4m3(blk)
    assert sb.tolist() == [1]


def test_indexer_query_is_the_matmul(oracle_lib):
    """Q^I = c^Q wq_b: numpy's matmul on the exact bf16 values, row 128 h + d
    of wq_b giving head h, dim d."""
    rng = np.random.default_rng(23)
    cq = g.f32_to_bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    wq = g.f32_to_bf16_bits(rng.standard_normal((256, 64)).astype(np.float32))
    q = oracle.indexer_query(cq, wq)
    ref = g.bf16_bits_to_f32(cq).astype(np.float64) @ g.bf16_bits_to_f32(wq).astype(np.float64).T
    np.testing.assert_allclose(q, ref, rtol=1e-12, atol=1e-12)
    assert q.reshape(3, 2, 128)[1, 1, 5] == q[1, 128 + 5]


def _kvb_from_explicit(W_UK, W_UV, H, Dn, Dv):
    """kv_b_proj's Linear weight [H (Dn + Dv), Dc] holding the step list's
    W_UK [Dc, H Dn] and W_UV [Dc, H Dv]: per head its Dn key rows, then its Dv
    value rows (heads x (key dims + value dims), the nnterp module tree)."""
    Dc = W_UK.shape[0]
    kvb = np.empty((H, Dn + Dv, Dc))
    kvb[:, :Dn] = W_UK.T.reshape(H, Dn, Dc)
    kvb[:, Dn:] = W_UV.T.reshape(H, Dv, Dc)
    return kvb.reshape(H * (Dn + Dv), Dc)


def test_absorption_routines_equal_explicit_form(oracle_lib):
    """absorb_query -> sparse attention -> absorb_output equals the explicit
    form with per-head keys c W_UK and values c W_UV (the oracle's explicit
    routine).  Inputs are multiples of 1/4 in [-3/4, 3/4], so the absorbed
    query and the fp32 storage the attention reads are exact: 1e-12."""
    rng = np.random.default_rng(30)
    H, Dc, Dn, Dv, Dr, S = 3, 16, 8, 6, 4, 11
    sm = 0.31
    q4 = lambda *shape: rng.integers(-3, 4, shape) / 4.0
    qb = q4(1, H, Dn + Dr)
    W_UK, W_UV = q4(Dc, H * Dn), q4(Dc, H * Dv)
    kvb = _kvb_from_explicit(W_UK, W_UV, H, Dn, Dv)
    kv = q4(S, Dc + Dr)
    cos0, sin0 = np.ones((1, Dr // 2)), np.zeros((1, Dr // 2))
    q = oracle.absorb_query(qb, kvb, cos0, sin0, Dn=Dn)
    # latent part: numpy's product of the head's W_UK block with q^C
    for h in range(H):
        np.testing.assert_allclose(q[0, h, :Dc], W_UK[:, h * Dn:(h + 1) * Dn] @ qb[0, h, :Dn],
                                   rtol=1e-12, atol=1e-12)
    # angle 0: the rotary part is q^pe's even dims, then its odd ones
    np.testing.assert_array_equal(q[0, :, Dc:Dc + Dr // 2], qb[0, :, Dn::2])
    np.testing.assert_array_equal(q[0, :, Dc + Dr // 2:], qb[0, :, Dn + 1::2])
    cfg = _cfg(B=1, T=1, S=S, H=H, Dc=Dc, Dr=Dr, K=S, sm_scale=sm)
    o_lat, _ = oracle.sparse_mla(cfg, [0], q.astype(np.float32), kv[None].astype(np.float32),
                                 np.arange(S, dtype=np.int32)[None])
    out = oracle.absorb_output(o_lat, kvb, Dn=Dn)
    explicit = oracle.explicit_mla(qb[0, :, :Dn], q[0, :, Dc:], kv[:, :Dc], kv[:, Dc:], W_UK, W_UV,
                                   np.float64(np.float32(sm)))
    np.testing.assert_allclose(out.reshape(H, Dv), explicit, rtol=1e-12, atol=1e-12)


def test_absorbed_query_rotation_matches_cached_key(oracle_lib):
    """The query's rotary part and the cached key's (cache_fill) turn alike:
    their dot product depends on the two angles' difference only, so
    q(a) . k(b) = q(a - b) . k(0) and q(a) . k(a) = q(0) . k(0)."""
    rng = np.random.default_rng(31)
    n, H = 4, 2
    # keys: a projection that passes x straight into the rotary block
    x = g.f32_to_bf16_bits(rng.standard_normal((n, 64)).astype(np.float32))
    W = np.zeros((768, 64), np.float32)
    W[512:576] = np.eye(64)
    W = g.f32_to_bf16_bits(W)
    a = rng.uniform(-math.pi, math.pi, (n, 32))
    b = rng.uniform(-math.pi, math.pi, (n, 32))
    f = lambda ang: (np.cos(ang), np.sin(ang))

    def key(ang):
        c, s = f(ang)
        kv, _, _ = oracle.cache_fill(x, W, np.ones(512), np.ones(128), np.zeros(128),
                                     c.astype(np.float32), s.astype(np.float32))
        return kv[:, 512:]

    qb = rng.standard_normal((n, H, 8 + 64))
    kvb = rng.standard_normal((H * 16, 4))

    def query(ang):
        c, s = f(ang)
        return oracle.absorb_query(qb, kvb, c, s, Dn=8)[:, :, 4:]

    dot = lambda q, k: np.einsum("nhd,nd->nh", q, k)
    np.testing.assert_allclose(dot(query(a), key(b)), dot(query(a - b), key(np.zeros_like(b))),
                               rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(dot(query(a), key(a)), dot(query(0 * a), key(0 * a)),
                               rtol=1e-6, atol=1e-6)


def test_linear_bf16_is_the_matmul(oracle_lib):
    """wo: numpy's matmul x W^T on the exact bf16 values (a non-square W)."""
    rng = np.random.default_rng(32)
    x = g.f32_to_bf16_bits(rng.standard_normal((3, 96)).astype(np.float32))
    W = g.f32_to_bf16_bits(rng.standard_normal((40, 96)).astype(np.float32))
    out = oracle.linear_bf16(x, W)
    ref = g.bf16_bits_to_f32(x).astype(np.float64) @ g.bf16_bits_to_f32(W).astype(np.float64).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)

"""GPU parity: every libdsa entry point against the CPU oracle (MI355X only).

Inputs are the seeded synthetic workloads of ``dsa_inputs`` (or small
variants of them), identical bytes on both sides.  The bar:
  * index scores: bit-exact on integer-valued inputs (sums are exact in fp32
    and fp64); otherwise within 1e-4 of the row's largest |score|;
  * top-K: bit-exact against the oracle's selection on the SAME fp32 scores;
    end to end (GPU scores vs oracle scores) a key may differ only within the
    1e-5 relative gap of the K-th score;
  * latent attention on the same indices: per (b, t, h) row within 1e-4
    (fp32) / 2e-2 (bf16) of the row's largest |o|; lse within the same bar
    in absolute terms.
"""
import math

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


def _rows(cfg, rows=None):
    if rows is None:
        rb = np.repeat(np.arange(cfg.B, dtype=np.int32), cfg.T)
        rt = np.tile(np.arange(cfg.T, dtype=np.int32), cfg.B)
    else:
        rb = np.array([r[0] for r in rows], np.int32)
        rt = np.array([r[1] for r in rows], np.int32)
    return rb, rt


def _host_rows(cfg, tensor, rb, rt):
    """Per-query rows of q_idx / w / q for the listed (b, t)."""
    parts = [g.rows(cfg, tensor, int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)]
    if isinstance(parts[0], tuple):
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    return np.concatenate(parts)


def _oracle_scores(cfg, rb, rt, seq_lens=None):
    k = g.full(cfg, "k_idx")
    qi = _host_rows(cfg, "q_idx", rb, rt)
    w = _host_rows(cfg, "w", rb, rt)
    if cfg.idx_dtype == "fp8":
        return oracle.indexer_scores(cfg, rb, rt, qi[0], w, k[0], qi[1], k[1], seq_lens=seq_lens)
    return oracle.indexer_scores(cfg, rb, rt, qi, w, k, seq_lens=seq_lens)


def _inputs(cfg):
    d = {n: U.upload(cfg, n) for n in ("q_idx", "k_idx", "w", "q", "kv")}
    if cfg.idx_dtype == "fp8":
        d["q_idx"], d["q_sf"] = d["q_idx"]
        d["k_idx"], d["k_sf"] = d["k_idx"]
    else:
        d["q_sf"] = d["k_sf"] = None
    return d


def _gpu_scores(dsa, cfg, x):
    return dsa.dsa_indexer_scores(U.shape_of(cfg), x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"])


# ---------------------------------------------------------------------------
# index scores
# ---------------------------------------------------------------------------

SCORE_CASES = {
    # generic VALU kernel (4 heads x 32 dims, fp32), integer inputs: bit-exact
    "tiny": g.CONFIGS["tiny"],
    # MFMA bf16 kernel, decode, integer twin: bit-exact
    "decode_int": g.CONFIGS["decode_8k"].replace(B=3, integer=True),
    # query-blocked MFMA bf16 kernel, causal prefill with ragged query blocks
    # and key chunks, integer: bit-exact
    "prefill_int": g.CONFIGS["prefill_16k"].replace(T=300, S=1000, integer=True),
    # the same kernel at its smallest T (one query block per sequence), fp32
    # head weights, S not a multiple of 4 (scalar fill of the future keys)
    "prefill_int_w32": g.CONFIGS["prefill_16k"].replace(B=3, T=8, S=517, w_dtype="f32",
                                                        integer=True),
    # one query short of it: the per-query kernel
    "prefill_int_t7": g.CONFIGS["prefill_16k"].replace(B=2, T=7, S=64, integer=True),
    # real-valued prefill, two sequences, T = S (every key chunk reaches the diagonal)
    "prefill_real": g.CONFIGS["prefill_16k"].replace(B=2, T=203, S=203),
    # MFMA e4m3 kernel, integer twin (scale byte 127): bit-exact
    "fp8_int": g.CONFIGS["decode_64k_fp8"].replace(B=2, S=4200, integer=True),
    # e4m3, three queries per sequence (causal tail), fp32 head weights, the
    # second key block holding one partial chunk
    "fp8_int_t3": g.CONFIGS["decode_64k_fp8"].replace(B=2, T=3, S=2100, w_dtype="f32",
                                                      integer=True),
    # e4m3, fewer keys than one chunk
    "fp8_int_short": g.CONFIGS["decode_64k_fp8"].replace(B=3, S=40, integer=True),
    # e4m3 with many queries per sequence (a prefill chunk): 16 and 300
    # queries over 1000 keys, every key chunk meeting the causal diagonal
    "fp8_int_t16": g.CONFIGS["decode_64k_fp8"].replace(B=2, T=16, S=1000, integer=True),
    "fp8_int_t300": g.CONFIGS["decode_64k_fp8"].replace(B=1, T=300, S=1000, integer=True),
    # the same with fp32 head weights and a sequence length that is not a
    # multiple of 4 (the per-query kernel), real-valued
    "fp8_real_t37": g.CONFIGS["decode_64k_fp8"].replace(B=2, T=37, S=517, w_dtype="f32"),
    # query-blocked e4m3 kernel, real-valued: the last 512 queries of 2048 keys,
    # and fp32 head weights with a ragged last query block and key chunk
    "fp8_real_t512": g.CONFIGS["decode_64k_fp8"].replace(B=1, T=512, S=2048),
    "fp8_real_w32_t70": g.CONFIGS["decode_64k_fp8"].replace(B=2, T=70, S=1300, w_dtype="f32"),
    # real-valued: within 1e-4 of the row max
    "decode_real": g.CONFIGS["decode_8k"].replace(B=2, S=3000),
    "fp8_real": g.CONFIGS["decode_64k_fp8"].replace(B=2, S=5000),
    # generic kernel on bf16 with odd sizes
    "generic_bf16": g.Config("generic_bf16", B=2, T=3, S=77, HI=5, DI=24, H=4, Dc=64, Dr=16, K=20,
                             idx_dtype="bf16", w_dtype="bf16", mla_dtype="bf16", seed=5),
}


@pytest.mark.parametrize("case", sorted(SCORE_CASES))
def test_indexer_scores(dsa, case):
    cfg = SCORE_CASES[case]
    print(f"[indexer_scores] {case}: {cfg}", flush=True)
    x = _inputs(cfg)
    got = _gpu_scores(dsa, cfg, x).cpu().numpy().reshape(cfg.B * cfg.T, cfg.S)
    rb, rt = _rows(cfg)
    ref = _oracle_scores(cfg, rb, rt)
    if cfg.integer:
        assert np.array_equal(got, ref), f"{case}: integer-valued scores must be bit-exact"
    else:
        U.assert_scores_close(got, ref, what=case)


# ragged batches: per-sequence context lengths, including one shorter than T
# (its first queries see nothing) and one of 0 keys; integer inputs: bit-exact
RAGGED_CASES = {
    "stream_decode": (g.CONFIGS["decode_8k"].replace(B=4, S=3000, integer=True),
                      [3000, 1700, 1, 0]),
    "stream_t3": (g.CONFIGS["decode_8k"].replace(B=3, T=3, S=2100, integer=True),
                  [2100, 1000, 2]),
    "stream_fp8": (g.CONFIGS["decode_64k_fp8"].replace(B=3, S=4200, integer=True),
                   [4200, 2049, 64]),
    "prefill": (g.CONFIGS["prefill_16k"].replace(B=3, T=300, S=1000, integer=True),
                [1000, 650, 100]),
    "prefill_fp8": (g.CONFIGS["decode_64k_fp8"].replace(B=3, T=20, S=1000, integer=True),
                    [1000, 500, 10]),
    "generic": (SCORE_CASES["generic_bf16"], [77, 30]),
}


@pytest.mark.parametrize("case", sorted(RAGGED_CASES))
def test_indexer_scores_ragged(dsa, case):
    cfg, lens = RAGGED_CASES[case]
    print(f"[indexer_scores_ragged] {case}: {cfg} lens={lens}", flush=True)
    torch = U.torch()
    x = _inputs(cfg)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    got = dsa.dsa_indexer_scores_ragged(U.shape_of(cfg), lens_dev, x["q_idx"], x["k_idx"], x["w"],
                                        x["q_sf"], x["k_sf"])
    got = got.cpu().numpy().reshape(cfg.B * cfg.T, cfg.S)
    rb, rt = _rows(cfg)
    ref = _oracle_scores(cfg, rb, rt, seq_lens=np.array(lens, np.int32))
    if cfg.integer:
        assert np.array_equal(got, ref), f"{case}: integer-valued scores must be bit-exact"
    else:
        assert np.array_equal(np.isfinite(got), np.isfinite(ref))
        U.assert_scores_close(got, ref, what=case)


# ---------------------------------------------------------------------------
# top-k on identical scores: bit-exact
# ---------------------------------------------------------------------------

def _special_rows(S, K, rng):
    rows = [rng.standard_normal(S).astype(np.float32),
            rng.integers(-3, 4, S).astype(np.float32),              # heavy ties
            np.zeros(S, np.float32),                                 # all equal
            np.where(rng.random(S) < 0.5, -0.0, 0.0).astype(np.float32),  # signed zeros
            np.full(S, -np.inf, np.float32)]                         # nothing selectable
    r = rng.standard_normal(S).astype(np.float32)
    r[rng.random(S) < 0.3] = np.nan
    r[rng.random(S) < 0.3] = -np.inf
    rows.append(r)
    r = rng.standard_normal(S).astype(np.float32)
    r[: S // 2] = -np.inf                                            # fewer than K selectable (for big K)
    rows.append(r)
    r = (rng.standard_normal(S) * 1e-30).astype(np.float32)          # subnormal-range values
    rows.append(r)
    r = rng.standard_normal(S).astype(np.float32)
    r[rng.choice(S, size=min(S, 3), replace=False)] = np.inf        # a few +inf: always selected
    rows.append(r)
    r = rng.integers(-2, 3, S).astype(np.float32)
    r[rng.random(S) < 0.5] = np.inf                                  # many tied +inf (lowest index wins)
    r[rng.random(S) < 0.1] = np.nan
    rows.append(r)
    return np.stack(rows)


# rows up to 32768 keys: one workgroup; longer rows: 16 K-key chunks (40000,
# 40001, 131072) or 32 K-key chunks (300000: 19 chunks x 2048 > 32768) and a
# merge; candidates that fit no merge: the long-row select over 4096-key
# chunks (600000 keys; K of 30000 over 100003 keys)
@pytest.mark.parametrize("S,K", [(256, 32), (1000, 64), (3000, 2048), (8192, 2048),
                                 (16384, 2048), (40000, 2048), (40001, 2048), (131072, 2048),
                                 (300000, 2048), (600000, 2048), (100003, 30000), (100, 300)])
def test_topk_bit_exact(dsa, S, K):
    print(f"[topk] S={S} K={K}", flush=True)
    torch = U.torch()
    rng = np.random.default_rng(S + K)
    sc = _special_rows(S, K, rng)
    cfg = g.CONFIGS["decode_8k"].replace(B=sc.shape[0], T=1, S=S, K=K)
    got = dsa.dsa_topk(U.shape_of(cfg), torch.from_numpy(sc).cuda().view(cfg.B, 1, S))
    got = got.cpu().numpy().reshape(cfg.B, -1)
    ref = oracle.topk(cfg, sc)
    for r in range(cfg.B):
        assert np.array_equal(got[r], ref[r]), f"row {r} differs"


def _long_rows(S, rng):
    rows = [rng.standard_normal(S).astype(np.float32)]                     # real-valued
    rows.append(rng.integers(-3, 4, S).astype(np.float32))                # heavy ties: split by index
    r = np.full(S, -np.inf, np.float32)
    r[rng.choice(S, size=1500, replace=False)] = rng.standard_normal(1500)  # fewer than K selectable
    rows.append(r)
    rows.append(np.full(S, 0.25, np.float32))                              # one value everywhere
    return np.stack(rows)


def test_topk_long_rows_reuse_workspace(dsa):
    """The long-row select's workgroups meet through tagged words of the
    workspace: from arbitrary bytes, three calls in a row on one workspace,
    each on other rows, each give the oracle's selection.  (K = 8192 over
    131077 keys: candidates that fit no merge; more pairs than the last
    workgroup holds in registers.)"""
    torch = U.torch()
    S, K = 131072 + 5, 8192
    cfg = g.CONFIGS["decode_8k"].replace(B=4, T=1, S=S, K=K)
    shape = U.shape_of(cfg)
    ws = torch.empty(dsa.workspace_bytes(shape, dsa.ENTRY_TOPK), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    for rep in range(3):
        print(f"[topk_long] reuse call {rep}", flush=True)
        sc = np.roll(_long_rows(S, np.random.default_rng(100 + rep)), rep, axis=0)
        got = dsa.dsa_topk(shape, torch.from_numpy(sc).cuda().view(cfg.B, 1, S), ws=ws)
        got = got.cpu().numpy().reshape(cfg.B, -1)
        assert np.array_equal(got, oracle.topk(cfg, sc)), f"call {rep} differs"


def test_topk_long_rows_graph_replay(dsa):
    """Captured once in a HIP graph (the call's tag fixed at capture), the
    long-row select gives the oracle's selection on every replay, with eager
    calls in between: the row's last workgroup marks its words stale.
    (K = 12000 over 70000 keys takes the long-row select.)"""
    torch = U.torch()
    S, K = 70000, 12000
    cfg = g.CONFIGS["decode_8k"].replace(B=4, T=1, S=S, K=K)
    shape = U.shape_of(cfg)
    sc = torch.from_numpy(_long_rows(S, np.random.default_rng(7))).cuda().view(cfg.B, 1, S)
    ws = torch.empty(dsa.workspace_bytes(shape, dsa.ENTRY_TOPK), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    out = torch.empty((cfg.B, 1, K), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dsa.dsa_topk(shape, sc, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dsa.dsa_topk(shape, sc, out=out, ws=ws)
    for rep in range(3):
        print(f"[topk_long] replay {rep}", flush=True)
        rows = np.roll(_long_rows(S, np.random.default_rng(200 + rep)), rep, axis=0)
        sc.copy_(torch.from_numpy(rows).view(cfg.B, 1, S))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.topk(cfg, rows)
        assert np.array_equal(out.cpu().numpy().reshape(cfg.B, -1), ref), f"replay {rep} differs"
        eager = dsa.dsa_topk(shape, sc)                  # the program's own work between replays
        torch.cuda.synchronize()
        assert np.array_equal(eager.cpu().numpy().reshape(cfg.B, -1), ref)


def _random_topk_case(rng):
    """One seeded (S, K, rows) case: lengths across the one-workgroup,
    two-stage and long-row plans, K from 1 to past S, value patterns from
    spread reals to heavy ties, NaN, -inf and +inf."""
    S = int(rng.choice([int(rng.integers(1, 4097)), int(rng.integers(4097, 32769)),
                        int(rng.integers(32769, 140000)), int(rng.integers(140000, 700000))]))
    K = int(rng.choice([int(rng.integers(1, 65)), 2048, int(rng.integers(1, 40000)), S + int(rng.integers(0, 9))]))
    B = int(rng.integers(1, 4))
    rows = []
    for _ in range(B):
        kind = int(rng.integers(0, 5))
        if kind == 0:
            r = rng.standard_normal(S).astype(np.float32)
        elif kind == 1:
            r = rng.integers(-4, 5, S).astype(np.float32)
        elif kind == 2:
            r = (rng.standard_normal(S) * 10 ** rng.uniform(-30, 30)).astype(np.float32)
        elif kind == 3:
            r = rng.standard_normal(S).astype(np.float32)
            r[rng.random(S) < 0.3] = -np.inf
            r[rng.random(S) < 0.1] = np.nan
            r[rng.random(S) < 0.001] = np.inf
        else:
            r = np.full(S, -np.inf, np.float32)
            n = int(rng.integers(0, min(S, 3000) + 1))
            r[rng.choice(S, size=n, replace=False)] = rng.integers(-2, 3, n).astype(np.float32)
        rows.append(r)
    return S, K, np.stack(rows)


@pytest.mark.parametrize("seed", range(24))
def test_topk_random_shapes(dsa, seed):
    """Seeded random shapes and value patterns: the selection equals the
    oracle's bit for bit whichever plan the shape takes."""
    torch = U.torch()
    S, K, sc = _random_topk_case(np.random.default_rng(1000 + seed))
    cfg = g.CONFIGS["decode_8k"].replace(B=sc.shape[0], T=1, S=S, K=K)
    print(f"[topk_random] seed={seed} B={cfg.B} S={S} K={K}", flush=True)
    got = dsa.dsa_topk(U.shape_of(cfg), torch.from_numpy(sc).cuda().view(cfg.B, 1, S))
    got = got.cpu().numpy().reshape(cfg.B, -1)
    ref = oracle.topk(cfg, sc)
    for r in range(cfg.B):
        assert np.array_equal(got[r], ref[r]), f"row {r} differs"


def test_topk_on_gpu_scores(dsa):
    """Selection from the GPU's own fp32 scores matches the oracle's selection
    of those same scores exactly (decode 8k shape, real-valued)."""
    cfg = g.CONFIGS["decode_8k"].replace(B=4)
    x = _inputs(cfg)
    sc = _gpu_scores(dsa, cfg, x)
    got = dsa.dsa_topk(U.shape_of(cfg), sc).cpu().numpy().reshape(cfg.B, -1)
    ref = oracle.topk(cfg, sc.cpu().numpy().reshape(cfg.B, -1))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# sparse latent attention on identical indices
# ---------------------------------------------------------------------------

def _mla_check(dsa, cfg, idx_np, rb, x=None):
    torch = U.torch()
    x = x or _inputs(cfg)
    idx = torch.from_numpy(idx_np.reshape(cfg.B, cfg.T, -1)).cuda()
    o, lse = dsa.dsa_sparse_mla_fwd(U.shape_of(cfg), x["q"], x["kv"], idx)
    o = U.dev_to_np(o, cfg.mla_dtype).reshape(cfg.B * cfg.T, cfg.H, cfg.Dc)
    if cfg.mla_dtype == "bf16":
        o = g.bf16_bits_to_f32(o)
    lse = lse.cpu().numpy().reshape(cfg.B * cfg.T, cfg.H)
    q = g.full(cfg, "q").reshape(cfg.B * cfg.T, cfg.H, cfg.D)
    kv = g.full(cfg, "kv")
    ro, rl = oracle.sparse_mla(cfg, rb, q, kv, idx_np.reshape(cfg.B * cfg.T, -1))
    U.assert_rows_close(o, ro, U.RTOL[cfg.mla_dtype], what=f"{cfg.name} o")
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(np.abs(lse[fin] - rl[fin]) <= U.RTOL[cfg.mla_dtype] * np.maximum(1, np.abs(rl[fin])))
    return o, lse


def _random_idx(cfg, rng, frac_invalid=0.0):
    W = cfg.K_eff
    rows = []
    for _ in range(cfg.B * cfg.T):
        sel = np.sort(rng.choice(cfg.S, size=W, replace=False)).astype(np.int32)
        if frac_invalid:
            sel[rng.random(W) < frac_invalid] = -1
        rows.append(sel)
    return np.stack(rows)


def _random_mla_case(rng, seed):
    """One seeded attention case: the generic fp32 kernels (tiny shapes) or
    the V3.2 MFMA kernel, B x T rows with K_eff from 1 to past 4096, each row
    sorted distinct keys, unsorted with duplicates, with out-of-range
    entries, empty, or ending in -1 padding."""
    base = "tiny" if rng.random() < 0.15 else "decode_8k"
    B, T = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    S = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 9000)), int(rng.integers(9000, 40000))]))
    K = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 2049)), 2048, S + 2]))
    if base == "tiny":
        S, K = min(S, 3000), min(K, 300)
    if min(K, S) > 4096:
        B, T = 1, min(T, 2)
    cfg = g.CONFIGS[base].replace(B=B, T=T, S=S, K=K, seed=seed + 3)
    W = cfg.K_eff
    rows = []
    for _ in range(B * T):
        kind = int(rng.integers(0, 5))
        if kind == 0:
            r = np.sort(rng.choice(S, size=W, replace=False)).astype(np.int32)
        elif kind == 1:
            r = rng.integers(0, S, W).astype(np.int32)
        elif kind == 2:
            r = rng.integers(-3, S + 3, W).astype(np.int32)
        elif kind == 3:
            r = np.full(W, -1, np.int32)
        else:
            r = np.sort(rng.choice(S, size=W, replace=False)).astype(np.int32)
            r[int(rng.integers(0, W + 1)):] = -1
        rows.append(r)
    return cfg, np.stack(rows)


@pytest.mark.parametrize("seed", range(12))
def test_mla_random_shapes(dsa, seed):
    """Seeded random attention shapes and index rows: o and lse within the
    bar of the oracle's."""
    cfg, idx_np = _random_mla_case(np.random.default_rng(90000 + seed), seed)
    print(f"[mla_random] seed={seed} {cfg.name} B={cfg.B} T={cfg.T} S={cfg.S} K={cfg.K}", flush=True)
    rb, _ = _rows(cfg)
    _mla_check(dsa, cfg, idx_np, rb, x={n: U.upload(cfg, n) for n in ("q", "kv")})


def test_mla_tiny_fp32(dsa):
    cfg = g.CONFIGS["tiny"]
    rb, rt = _rows(cfg)
    idx = oracle.topk(cfg, _oracle_scores(cfg, rb, rt))
    _mla_check(dsa, cfg, idx, rb)


@pytest.mark.parametrize("B", [1, 4, 32])
def test_mla_mfma_decode(dsa, B):
    """MFMA kernel, decode split-K (B=1: 16-way ... B=32: 8-way) + combine."""
    cfg = g.CONFIGS["decode_8k"].replace(B=B)
    rb, _ = _rows(cfg)
    _mla_check(dsa, cfg, _random_idx(cfg, np.random.default_rng(B)), rb)


@pytest.mark.parametrize("B,K", [(8, 64), (3, 2048)])
def test_mla_mfma_head_halves(dsa, B, K):
    """Few query rows: two 2-wave workgroups of 64 heads per split (B=8, K=64:
    one split, so each writes its heads of o directly; B=3: 16 splits and the
    merge)."""
    cfg = g.CONFIGS["decode_8k"].replace(B=B, K=K)
    rb, _ = _rows(cfg)
    _mla_check(dsa, cfg, _random_idx(cfg, np.random.default_rng(100 + B)), rb)


def test_mla_mfma_prefill_rows(dsa):
    """MFMA kernel without splits (many query rows), causal-style short rows."""
    cfg = g.CONFIGS["prefill_16k"].replace(T=300, S=2500)
    rb, rt = _rows(cfg)
    idx = oracle.topk(cfg, _oracle_scores(cfg, rb, rt))
    _mla_check(dsa, cfg, idx, rb)


def test_mla_mfma_edge_indices(dsa):
    """-1 and out-of-range entries skipped, duplicates counted, empty rows give
    o = 0 and lse = -inf, a ragged last tile."""
    cfg = g.CONFIGS["decode_8k"].replace(B=6, S=4096, K=1000)
    rng = np.random.default_rng(7)
    idx = _random_idx(cfg, rng, frac_invalid=0.3)
    idx[1, :] = -1                                     # empty row
    idx[2, 5:] = -1                                    # five keys
    idx[3, :500] = idx[3, 0]                           # one key many times
    idx[4, ::7] = cfg.S + 5                            # out of range
    idx[5, :] = rng.integers(0, 3, cfg.K_eff)          # three keys, heavy duplicates
    rb, _ = _rows(cfg)
    o, lse = _mla_check(dsa, cfg, idx, rb)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def _kv_log2_logit(cfg, q_row, kv_rows):
    """sm_scale * q . kv_j in log2 units, fp64, for the keys kv_rows [n, D]."""
    return cfg.softmax_scale * (kv_rows.astype(np.float64) @ q_row.astype(np.float64)) / math.log(2.0)


def _plant_spikes(cfg, idx, q, kv, plants):
    """Replace the key row selected at position j of query row r by 8 q[r, h]
    (bf16): head h's logit for it then exceeds every other by far.  plants:
    (query row, batch, position j, head, first position of j's split).
    Returns the patched kv and, per plant, how far (log2 units) the spike's
    logit lies above the largest logit, for its head, of the 32 positions that
    open its split (the tile that sets the kernel's reference maximum)."""
    kv = kv.copy()
    for r, b, j, h, _ in plants:
        s = int(idx[r, j])
        kv[b, s] = g.f32_to_bf16_bits((8.0 * g.bf16_bits_to_f32(q[r, h])).astype(np.float32))
    gaps = []
    for r, b, j, h, first in plants:
        qr = g.bf16_bits_to_f32(q[r, h])
        keys = idx[r, first:first + 32]
        keys = keys[keys >= 0]
        ref = _kv_log2_logit(cfg, qr, g.bf16_bits_to_f32(kv[b, keys])).max()
        spike = _kv_log2_logit(cfg, qr, g.bf16_bits_to_f32(kv[b, idx[r, j]][None]))[0]
        gaps.append(spike - ref)
    return kv, gaps


@pytest.mark.parametrize("case", ["decode_split", "rows_window_reload"])
def test_mla_softmax_restart(dsa, case):
    """A selected key whose logit exceeds the largest logit of its split's
    first tile by more than 2^32 (an attention-sink-like spike): the kernel's
    fixed reference maximum no longer bounds the exponentials, so the split is
    run again with its true maximum.  decode_split: the decode shape with 4
    query rows (16 splits of 128 entries), spikes in late tiles of several
    splits, one row without.  rows_window_reload: 256 query rows of 2048
    selected keys each (no split; the index list passes through LDS in
    windows of 1024 entries, so the second pass starts by reloading the
    first window), spikes in the second window and in the first one.  The
    definition is unchanged by the spike: softmax over the selection."""
    torch = U.torch()
    if case == "decode_split":
        cfg = g.CONFIGS["decode_8k"].replace(B=4)
        rows, split = cfg.B, 128
        idx = _random_idx(cfg, np.random.default_rng(41))
        # (row, batch, position, head); the first tile of each split starts at
        # the split's first position
        plants = [(0, 0, 70, 5), (1, 1, 5 * 128 + 100, 77), (2, 2, 2047, 127)]
    else:
        cfg = g.CONFIGS["prefill_16k"].replace(B=1, T=256, S=4096)
        rows, split = cfg.T, cfg.K_eff
        idx = _random_idx(cfg, np.random.default_rng(42))
        plants = [(3, 0, 1500, 0), (200, 0, 40, 64), (255, 0, 2047, 100)]
    print(f"[mla_softmax_restart] {case}: {cfg}", flush=True)
    q = g.full(cfg, "q").reshape(rows, cfg.H, cfg.D)
    kv = g.full(cfg, "kv")
    kv, gaps = _plant_spikes(cfg, idx, q, kv, [p + (p[2] // split * split,) for p in plants])
    assert min(gaps) > 32.0, f"spikes do not reach the restart condition: {gaps}"
    dev_q = U.to_dev(q.reshape(cfg.B, cfg.T, cfg.H, cfg.D), "bf16")
    dev_kv = U.to_dev(kv, "bf16")
    o, lse = dsa.dsa_sparse_mla_fwd(U.shape_of(cfg), dev_q, dev_kv,
                                    torch.from_numpy(idx.reshape(cfg.B, cfg.T, -1)).cuda())
    o = g.bf16_bits_to_f32(U.dev_to_np(o, "bf16")).reshape(rows, cfg.H, cfg.Dc)
    lse = lse.cpu().numpy().reshape(rows, cfg.H)
    rb, _ = _rows(cfg)
    ro, rl = oracle.sparse_mla(cfg, rb, q, kv, idx)
    U.assert_rows_close(o, ro, U.RTOL["bf16"], what=f"{case} o")
    assert np.all(np.abs(lse - rl) <= U.RTOL["bf16"] * np.maximum(1, np.abs(rl)))
    for r, b, j, h in plants:  # the spike's head puts (almost) all its weight on the spike
        spike = g.bf16_bits_to_f32(kv[b, idx[r, j], :cfg.Dc])
        assert np.abs(o[r, h] - spike).max() <= U.RTOL["bf16"] * np.abs(spike).max()


def test_mla_generic_bf16(dsa):
    cfg = SCORE_CASES["generic_bf16"]
    rb, _ = _rows(cfg)
    _mla_check(dsa, cfg, _random_idx(cfg, np.random.default_rng(3), 0.2), rb)


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------

def _forward(dsa, cfg, x):
    o, lse, idx = dsa.dsa_forward(U.shape_of(cfg), x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                  x["q_sf"], x["k_sf"])
    return o, lse, idx


def test_forward_tiny_exact_selection(dsa):
    cfg = g.CONFIGS["tiny"]
    x = _inputs(cfg)
    o, lse, idx = _forward(dsa, cfg, x)
    rb, rt = _rows(cfg)
    ref_idx = oracle.topk(cfg, _oracle_scores(cfg, rb, rt))
    assert np.array_equal(idx.cpu().numpy().reshape(cfg.T, -1), ref_idx)
    ro, rl = oracle.sparse_mla(cfg, rb, g.full(cfg, "q")[0], g.full(cfg, "kv"), ref_idx)
    U.assert_rows_close(o.cpu().numpy().reshape(cfg.T, cfg.H, cfg.Dc), ro, U.RTOL["f32"], "tiny o")


def test_forward_at_the_row_limit(dsa):
    """65535 query rows (257 sequences x 255 queries), the most one call takes:
    every grid's row dimension at its limit (generic indexer, top-K, generic
    attention), integer inputs, selection and scores exact."""
    cfg = g.CONFIGS["tiny"].replace(B=257, T=255)
    assert cfg.B * cfg.T == 65535
    x = _inputs(cfg)
    o, lse, idx = _forward(dsa, cfg, x)
    rows = cfg.B * cfg.T
    rb, rt = _rows(cfg)
    ref_sc = oracle.indexer_scores(cfg, rb, rt, g.full(cfg, "q_idx").reshape(rows, cfg.HI, cfg.DI),
                                   g.full(cfg, "w").reshape(rows, cfg.HI), g.full(cfg, "k_idx"))
    ref_idx = oracle.topk(cfg, ref_sc)
    assert np.array_equal(idx.cpu().numpy().reshape(rows, -1), ref_idx)
    ro, rl = oracle.sparse_mla(cfg, rb, g.full(cfg, "q").reshape(rows, cfg.H, cfg.D), g.full(cfg, "kv"), ref_idx)
    U.assert_rows_close(o.cpu().numpy().reshape(rows, cfg.H, cfg.Dc), ro, U.RTOL["f32"], "row limit o")


def test_forward_dense_when_k_covers_causal(dsa):
    """K >= causal length: the sparse path is plain causal attention."""
    cfg = g.CONFIGS["tiny"].replace(K=256)
    x = _inputs(cfg)
    o, lse, idx = _forward(dsa, cfg, x)
    rb, rt = _rows(cfg)
    idx = idx.cpu().numpy().reshape(cfg.T, -1)
    assert np.array_equal((idx >= 0).sum(1), rt + 1)
    do, dl = oracle.dense_mla(cfg, rb, rt, g.full(cfg, "q")[0], g.full(cfg, "kv"))
    U.assert_rows_close(o.cpu().numpy().reshape(cfg.T, cfg.H, cfg.Dc), do, U.RTOL["f32"], "dense")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(cfg.T, cfg.H), dl, rtol=1e-5, atol=1e-5)


def test_forward_ragged(dsa):
    """A ragged decode batch: short sequences select fewer than K keys (their
    rows end in -1) and attend over their own keys only."""
    cfg = g.CONFIGS["decode_8k"].replace(B=4, S=3000)
    lens = [3000, 2500, 1000, 37]
    torch = U.torch()
    x = _inputs(cfg)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse, idx = dsa.dsa_forward_ragged(U.shape_of(cfg), lens_dev, x["q_idx"], x["k_idx"], x["w"],
                                         x["q"], x["kv"], x["q_sf"], x["k_sf"])
    rb, rt = _rows(cfg)
    ref_sc = _oracle_scores(cfg, rb, rt, seq_lens=np.array(lens, np.int32))
    ref_idx = oracle.topk(cfg, ref_sc)
    idx = idx.cpu().numpy().reshape(cfg.B, -1)
    U.assert_selection_within_gap(idx, ref_idx, ref_sc)
    for b, L in enumerate(lens):
        assert (idx[b] >= 0).sum() == min(L, cfg.K_eff)
        assert idx[b][idx[b] >= 0].max() < L
    ro, rl = oracle.sparse_mla(cfg, rb, g.full(cfg, "q").reshape(cfg.B, cfg.H, cfg.D),
                               g.full(cfg, "kv"), idx)
    o = g.bf16_bits_to_f32(U.dev_to_np(o, "bf16")).reshape(cfg.B, cfg.H, cfg.Dc)
    U.assert_rows_close(o, ro, U.RTOL["bf16"], "ragged o")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(cfg.B, cfg.H), rl, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("name,over,lens", [
    ("prefill_16k", dict(T=300, S=300), None),                       # T = S: row t sees t + 1 keys
    ("prefill_16k", dict(T=40, S=2500), None),                       # S > T: row t sees S - T + t + 1
    ("prefill_16k_fp8", dict(T=40, S=2500), None),
    ("prefill_16k", dict(B=3, T=40, S=2500), [2500, 1200, 20]),      # ragged: the last has rows that see nothing
    ("prefill_16k", dict(T=8, S=70000), None),                       # rows past one workgroup: two-stage top-K
    ("prefill_16k", dict(T=8, S=70000, K=12000), None),              # candidates that fit no merge: long rows
])
def test_forward_reads_only_visible_scores(dsa, name, over, lens):
    """Inside dsa_forward the many-query indexer leaves a causal row's
    invisible keys unwritten and the top-K ignores each row past its query's
    position: with the workspace filled with 0x7f bytes (each an unwritten
    score of 3.4e38, which would be selected if it counted), the selection is
    still the oracle's, exactly (integer twins)."""
    torch = U.torch()
    cfg = g.CONFIGS[name].replace(integer=True, **over)
    print(f"[forward_visible] {cfg.name} {over} lens={lens}", flush=True)
    x = _inputs(cfg)
    shape = U.shape_of(cfg)
    ws = torch.full((dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD),), 0x7F, dtype=torch.uint8, device="cuda")
    lens_dev = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, _, idx = dsa.dsa_forward_ragged(shape, lens_dev, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                       x["q_sf"], x["k_sf"], ws=ws)
    rb, rt = _rows(cfg)
    ref_sc = _oracle_scores(cfg, rb, rt, seq_lens=None if lens is None else np.array(lens, np.int32))
    got = idx.cpu().numpy().reshape(cfg.B * cfg.T, -1)
    assert np.array_equal(got, oracle.topk(cfg, ref_sc))


def _random_forward_case(rng, seed):
    """One seeded dsa_forward shape: bf16 or e4m3 indexer, T from 1 (the
    streaming kernels) to 48 (the many-query kernels), S up to 45000 (past
    one top-K workgroup), K small, 2048 or past S, full or ragged contexts
    (lengths 0 .. S); integer twins, so the selection is exact."""
    base = "prefill_16k_fp8" if rng.random() < 0.4 else "prefill_16k"
    B = int(rng.integers(1, 4))
    S = int(rng.choice([int(rng.integers(1, 600)), int(rng.integers(600, 5000)),
                        int(rng.integers(33000, 45000))]))
    T = int(rng.integers(1, min(S, 48) + 1))
    K = int(rng.choice([int(rng.integers(1, 64)), 2048, S + 3]))
    if S > 30000:
        B, T = 1, int(rng.integers(1, 9))
    cfg = g.CONFIGS[base].replace(B=B, T=T, S=S, K=K, integer=True, seed=seed + 1)
    lens = [int(rng.integers(0, S + 1)) for _ in range(B)] if rng.random() < 0.5 else None
    return cfg, lens


@pytest.mark.parametrize("seed", range(16))
def test_forward_random_shapes(dsa, seed):
    """Seeded random dsa_forward shapes over a workspace of 0x7f bytes: the
    selection equals the oracle's top-K of the oracle's scores, exactly."""
    torch = U.torch()
    cfg, lens = _random_forward_case(np.random.default_rng(70000 + seed), seed)
    print(f"[forward_random] seed={seed} {cfg.name} B={cfg.B} T={cfg.T} S={cfg.S} K={cfg.K} lens={lens}",
          flush=True)
    x = _inputs(cfg)
    shape = U.shape_of(cfg)
    ws = torch.full((max(1, dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD)),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    lens_dev = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, _, idx = dsa.dsa_forward_ragged(shape, lens_dev, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                       x["q_sf"], x["k_sf"], ws=ws)
    rb, rt = _rows(cfg)
    ref_sc = _oracle_scores(cfg, rb, rt, seq_lens=None if lens is None else np.array(lens, np.int32))
    got = idx.cpu().numpy().reshape(cfg.B * cfg.T, -1)
    assert np.array_equal(got, oracle.topk(cfg, ref_sc))


FORWARD_CASES = {
    "decode_int": g.CONFIGS["decode_8k"].replace(B=4, integer=True),
    "decode_real": g.CONFIGS["decode_8k"].replace(B=4),
    # two queries per sequence (the multi-token-prediction decode step): the
    # second query also sees the first one's position
    "decode_mtp": g.CONFIGS["decode_8k"].replace(B=2, T=2, S=3000),
    # the YaRN-scaled softmax scale of the nnterp page (0.1352) instead of
    # 1/sqrt(192)
    "decode_yarn": g.CONFIGS["decode_8k"].replace(B=2, S=3000, sm_scale=0.1352),
    # fewer keys than K: every key is selected, the sparse path is dense MLA
    "decode_dense": g.CONFIGS["decode_8k"].replace(B=2, S=1500),
    # the e4m3 indexer in front of the attention
    "decode_fp8": g.CONFIGS["decode_64k_fp8"].replace(B=2, S=5000),
}


@pytest.mark.parametrize("case", sorted(FORWARD_CASES))
def test_forward_decode(dsa, case):
    cfg = FORWARD_CASES[case]
    print(f"[forward] {case}: {cfg}", flush=True)
    x = _inputs(cfg)
    o, lse, idx = _forward(dsa, cfg, x)
    rb, rt = _rows(cfg)
    rows = cfg.B * cfg.T
    ref_sc = _oracle_scores(cfg, rb, rt)
    ref_idx = oracle.topk(cfg, ref_sc)
    idx = idx.cpu().numpy().reshape(rows, -1)
    if cfg.integer:
        assert np.array_equal(idx, ref_idx)
    else:
        U.assert_selection_within_gap(idx, ref_idx, ref_sc)
    if cfg.K >= cfg.S:
        assert np.array_equal(idx, np.tile(np.arange(cfg.S, dtype=np.int32), (rows, 1)))
    ro, rl = oracle.sparse_mla(cfg, rb, g.full(cfg, "q").reshape(rows, cfg.H, cfg.D),
                               g.full(cfg, "kv"), idx)
    o = g.bf16_bits_to_f32(U.dev_to_np(o, "bf16")).reshape(rows, cfg.H, cfg.Dc)
    U.assert_rows_close(o, ro, U.RTOL["bf16"], f"{case} o")
    np.testing.assert_allclose(lse.cpu().numpy().reshape(rows, cfg.H), rl, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("name", ["decode_8k", "decode_128k", "decode_64k_fp8"])
def test_forward_bitwise_deterministic(dsa, name):
    """dsa_forward at the full decode shapes, twice on the same inputs, the
    second time with the workspace filled with random bytes: o, lse and the
    selection are identical bit for bit (fixed reduction orders everywhere, no
    atomics in the arithmetic, nothing read from the workspace before the call
    writes it).  Inputs are drawn on the GPU from a seeded generator."""
    torch = U.torch()
    cfg = g.CONFIGS[name]
    print(f"[forward_deterministic] {name}: {cfg}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(17)
    bf = lambda *shape: torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    if cfg.idx_dtype == "fp8":
        q_idx = torch.randint(0, 0x7F, (cfg.B, cfg.T, cfg.HI, cfg.DI), generator=gen, device="cuda",
                              dtype=torch.uint8) | (torch.randint(0, 2, (cfg.B, cfg.T, cfg.HI, cfg.DI),
                                                    generator=gen, device="cuda", dtype=torch.uint8) << 7)
        k_idx = torch.randint(0, 0x7F, (cfg.B, cfg.S, cfg.DI), generator=gen, device="cuda",
                              dtype=torch.uint8)
        q_sf = torch.randint(120, 130, (cfg.B, cfg.T, cfg.HI, 1), generator=gen, device="cuda",
                             dtype=torch.uint8)
        k_sf = torch.randint(120, 130, (cfg.B, cfg.S, 1), generator=gen, device="cuda", dtype=torch.uint8)
    else:
        q_idx, k_idx = bf(cfg.B, cfg.T, cfg.HI, cfg.DI), bf(cfg.B, cfg.S, cfg.DI)
        q_sf = k_sf = None
    w = bf(cfg.B, cfg.T, cfg.HI)
    q, kv = bf(cfg.B, cfg.T, cfg.H, cfg.D), bf(cfg.B, cfg.S, cfg.D)
    shape = U.shape_of(cfg)
    ws = torch.zeros(dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD), dtype=torch.uint8, device="cuda")
    o1, l1, i1 = dsa.dsa_forward(shape, q_idx, k_idx, w, q, kv, q_sf, k_sf, ws=ws)
    o1, l1, i1 = o1.clone(), l1.clone(), i1.clone()
    ws.copy_(torch.randint(0, 256, ws.shape, generator=gen, device="cuda", dtype=torch.uint8))
    o2, l2, i2 = dsa.dsa_forward(shape, q_idx, k_idx, w, q, kv, q_sf, k_sf, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2), "selection differs between runs"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "o differs between runs"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs between runs"
    assert bool((i1 >= 0).all()), "every decode row selects K keys"


def test_binding_rejects_bad_outputs(dsa):
    """The binding checks caller-supplied outputs and workspaces of
    dsa_forward before anything reaches the library (no launch happens)."""
    torch = U.torch()
    cfg = g.CONFIGS["decode_8k"].replace(B=2, S=3000)
    x = _inputs(cfg)
    shape = U.shape_of(cfg)
    args = (shape, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"])
    bad = [
        dict(out=torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dc - 1), dtype=torch.bfloat16, device="cuda")),
        dict(out=torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dc), dtype=torch.float32, device="cuda")),
        dict(idx_out=torch.empty((cfg.B, cfg.T, cfg.K_eff - 1), dtype=torch.int32, device="cuda")),
        dict(idx_out=torch.empty((cfg.B, cfg.T, cfg.K_eff), dtype=torch.int64, device="cuda")),
        dict(lse=torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")),
        dict(lse=torch.empty((cfg.B, cfg.T, cfg.H + 1), dtype=torch.float32, device="cuda")),
        dict(ws=torch.empty(dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD) // 4 + 1, dtype=torch.float32,
                            device="cuda")),
        dict(ws=torch.empty(2 * dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD), dtype=torch.uint8,
                            device="cuda")[::2]),
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            dsa.dsa_forward(*args, **kw)


# ---------------------------------------------------------------------------
# the fused index scores -> top-K of dsa_forward (decode shapes)
# ---------------------------------------------------------------------------

FUSED_CASES = {
    "decode_real": g.CONFIGS["decode_8k"].replace(B=8),
    # integer inputs: many equal scores, the boundary key exact with ties
    "decode_int": g.CONFIGS["decode_8k"].replace(B=8, integer=True),
    "mtp_t2": g.CONFIGS["decode_8k"].replace(B=2, T=2, S=3000),
    # a row length that is not a multiple of 4 (scalar reads of the row)
    "odd_keys": g.CONFIGS["decode_8k"].replace(B=3, S=3001),
    # fewer keys than K: every selectable key is taken
    "short_rows": g.CONFIGS["decode_8k"].replace(B=2, S=1500),
    "fp8_int": g.CONFIGS["decode_64k_fp8"].replace(B=3, S=20000, integer=True),
    "fp8_real": g.CONFIGS["decode_64k_fp8"].replace(B=3, S=20000),
    # 128 key blocks meeting per row, integer ties (no planted cluster: its
    # offsets are not integers)
    "long_int": g.CONFIGS["decode_128k"].replace(B=2, integer=True, cluster=0),
    # the planted cluster
    "long_real": g.CONFIGS["decode_128k"].replace(B=2),
}


@pytest.mark.parametrize("case", sorted(FUSED_CASES))
def test_fused_selection_exact(dsa, case):
    """dsa_indexer_topk selects inside the indexer launch: its selection
    equals the oracle's top-K of the very scores the launch left in the
    workspace, bit for bit, and those scores are the oracle's (exactly on
    integer inputs, within the score bar otherwise).  The workspace starts
    out holding arbitrary bytes, and the call runs twice on it."""
    torch = U.torch()
    cfg = FUSED_CASES[case]
    print(f"[fused_selection] {case}: {cfg}", flush=True)
    x = _inputs(cfg)
    shape = U.shape_of(cfg)
    ws = torch.empty(dsa.workspace_bytes(shape, dsa.ENTRY_INDEXER_TOPK), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                                       # whatever the workspace held before
    rows = cfg.B * cfg.T
    rb, rt = _rows(cfg)
    ref = _oracle_scores(cfg, rb, rt)
    first = None
    for rep in range(2):
        idx = dsa.dsa_indexer_topk(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"], ws=ws)
        torch.cuda.synchronize()
        sc = ws[: rows * cfg.S * 4].view(torch.float32).cpu().numpy().reshape(rows, cfg.S)
        got = idx.cpu().numpy().reshape(rows, -1)
        assert np.array_equal(got, oracle.topk(cfg, sc)), f"{case}: selection differs from the oracle's"
        if cfg.integer:
            assert np.array_equal(sc, ref)
        else:
            U.assert_scores_close(sc, ref, what=case)
        if first is None:
            first = got
        else:
            assert np.array_equal(first, got), f"{case}: the second call selects differently"


def test_fused_selection_ragged(dsa):
    """dsa_indexer_topk over a ragged batch (a sequence shorter than K, one
    with a single key, one with none): the oracle's selection of the scores
    it computed."""
    torch = U.torch()
    cfg = g.CONFIGS["decode_8k"].replace(B=4, S=3000, integer=True)
    lens = [3000, 1700, 1, 0]
    x = _inputs(cfg)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    shape = U.shape_of(cfg)
    ws = torch.empty(dsa.workspace_bytes(shape, dsa.ENTRY_INDEXER_TOPK), dtype=torch.uint8, device="cuda")
    idx = dsa.dsa_indexer_topk(shape, x["q_idx"], x["k_idx"], x["w"], seq_lens=lens_dev, ws=ws)
    rb, rt = _rows(cfg)
    ref_sc = _oracle_scores(cfg, rb, rt, seq_lens=np.array(lens, np.int32))
    assert np.array_equal(idx.cpu().numpy().reshape(cfg.B, -1), oracle.topk(cfg, ref_sc))

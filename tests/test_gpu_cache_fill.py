"""GPU parity of the cache fill and indexer inputs (dsa_cache_fill) against
the oracle (fp64).  Inputs are seeded draws: hidden states N(0, 1), the
joint projection N(0, 1/D) (so projections are O(1)), gains around 1, biases
around 0, rotation angles uniform.  bf16 outputs are compared row by row to
the oracle rounded once; E4M3 keys by their codes (equal except where the
oracle's fp64 value sits on a rounding tie of the GPU's fp32 one) and their
scale bytes."""
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


def _draw(N, D, seed):
    rng = np.random.default_rng(seed)
    x = g.f32_to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32))
    W = g.f32_to_bf16_bits((rng.standard_normal((768, D)) / math.sqrt(D)).astype(np.float32))
    kv_gamma = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    k_gamma = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    k_beta = (0.1 * rng.standard_normal(128)).astype(np.float32)
    ang = rng.uniform(-math.pi, math.pi, (N, 32))
    return dict(x=x, W=W, kv_gamma=kv_gamma, k_gamma=k_gamma, k_beta=k_beta,
                cos=np.cos(ang).astype(np.float32), sin=np.sin(ang).astype(np.float32))


def _run(dsa, d, slots, rows, kv_dt, k_dt, w_dt):
    torch = U.torch()
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = t(d["x"].view(np.int16)).view(torch.bfloat16)
    W = t(d["W"].view(np.int16)).view(torch.bfloat16)
    kv_cache = torch.full((rows, 576), 7.0, dtype=kv_dt, device=dev)
    if k_dt == "fp8":
        k_cache = torch.full((rows, 128), 0x55, dtype=torch.uint8, device=dev)
        k_sf = torch.full((rows,), 0xAA, dtype=torch.uint8, device=dev)
    else:
        k_cache = torch.full((rows, 128), 7.0, dtype=k_dt, device=dev)
        k_sf = None
    w = dsa.dsa_cache_fill(x, W, t(d["kv_gamma"]), t(d["k_gamma"]), t(d["k_beta"]), t(d["cos"]),
                           t(d["sin"]), t(np.asarray(slots, np.int64)), kv_cache, k_cache, k_sf,
                           w_dtype=w_dt)
    torch.cuda.synchronize()
    return kv_cache, k_cache, k_sf, w


def _host(tensor):
    torch = U.torch()
    if tensor.dtype == torch.bfloat16:
        return g.bf16_bits_to_f32(tensor.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return tensor.cpu().numpy().astype(np.float64)


def _rows_close(got, ref, rtol, what):
    err = np.abs(got - ref).max(axis=1)
    lim = rtol * np.abs(ref).max(axis=1)
    bad = np.nonzero(err > lim)[0]
    assert bad.size == 0, f"{what}: rows {bad[:5]} off by {err[bad[:5]]} (allowed {lim[bad[:5]]})"


def _check_fp8(codes, sb, ref):
    """GPU E4M3 rows vs the oracle's fp64 rows: the scale byte is the
    oracle's unless the row maximum is within 1e-5 of a scale boundary; codes
    equal the oracle's quantisation except on a near-tie, where the fp32
    accumulation over the hidden dimension (errors of about 1e-5 of the row's
    largest value) may land on the other side: there the two codes must be
    neighbours with the value within 2e-5 of the row maximum of their
    midpoint."""
    ref_codes, ref_sb = oracle.quantize_e4m3(ref)
    ref_sb = ref_sb[:, 0]
    amax = np.abs(ref).max(axis=1)
    ratio = np.log2(amax / 448.0)
    near_edge = np.abs(ratio - np.round(ratio)) < 1e-5
    assert np.all((sb == ref_sb) | near_edge), "scale bytes differ away from a boundary"
    ok = sb == ref_sb
    scaled = ref[ok] / np.exp2(ref_sb[ok].astype(np.float64) - 127)[:, None]
    deq_ref = g.e4m3_to_f32(ref_codes[ok]).astype(np.float64)
    diff = codes[ok] != ref_codes[ok]
    if diff.any():
        # a code may differ only where the value is (almost) half-way between two codes
        nxt = g.e4m3_to_f32(codes[ok]).astype(np.float64)
        mid = 0.5 * (nxt + deq_ref)
        step = np.abs(nxt - deq_ref)
        row_max = np.broadcast_to(np.abs(scaled).max(axis=1, keepdims=True), scaled.shape)
        assert np.all(np.abs(scaled[diff] - mid[diff]) <= 2e-5 * row_max[diff]), \
            "E4M3 codes differ away from a rounding tie"
        # neighbours: no representable value lies strictly between the two codes
        lo, hi = np.minimum(nxt, deq_ref)[diff], np.maximum(nxt, deq_ref)[diff]
        grid = g.e4m3_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
        grid = grid[np.isfinite(grid)]
        assert not np.any((grid[None, :] > lo[:, None]) & (grid[None, :] < hi[:, None]))
    assert diff.mean() < 1e-3


CASES = {
    # decode step: one token per sequence of a 32-sequence batch, V3.2 width
    "decode_bf16": (32, 7168, "bf16", "bf16", "bf16", 1),
    "decode_fp8_key": (32, 7168, "bf16", "fp8", "bf16", 2),
    # ragged token counts (partial 32-token blocks), fp32 outputs
    "tokens_70_f32": (70, 7168, "f32", "f32", "f32", 3),
    "tokens_5_fp8_small_width": (5, 256, "bf16", "fp8", "f32", 4),
    # enough tokens for the tiled kernel (128 x 128 tiles), a partial last tile
    "tokens_6000_tiled": (6000, 7168, "bf16", "fp8", "bf16", 5),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_cache_fill(dsa, case):
    N, D, kv_s, k_s, w_s, seed = CASES[case]
    print(f"[cache_fill] {case}: N={N} D={D} kv={kv_s} k={k_s} w={w_s}", flush=True)
    torch = U.torch()
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": "fp8"}
    d = _draw(N, D, seed)
    rows = 3 * N + 5
    rng = np.random.default_rng(seed + 100)
    slots = rng.permutation(rows)[:N].astype(np.int64)
    slots[N // 2] = -1                             # this token's cache writes are skipped
    kv_c, k_c, k_sf, w = _run(dsa, d, slots, rows, dt[kv_s], dt[k_s], dt[w_s])
    rkv, rk, rw = oracle.cache_fill(d["x"], d["W"], d["kv_gamma"], d["k_gamma"], d["k_beta"],
                                    d["cos"], d["sin"])
    live = slots >= 0
    rtol = 1e-2 if kv_s == "bf16" else 1e-4
    kv_h = _host(kv_c)
    _rows_close(kv_h[slots[live], :512], rkv[live, :512], rtol, "normalised latent")
    _rows_close(kv_h[slots[live], 512:], rkv[live, 512:], rtol, "rotated key")
    untouched = np.setdiff1d(np.arange(rows), slots[live])
    assert np.all(kv_h[untouched] == 7.0), "rows outside the slots must stay untouched"
    if k_s == "fp8":
        codes = k_c.cpu().numpy()
        sb = k_sf.cpu().numpy()
        _check_fp8(codes[slots[live]], sb[slots[live]], rk[live])
        assert np.all(codes[untouched] == 0x55) and np.all(sb[untouched] == 0xAA)
    else:
        k_h = _host(k_c)
        _rows_close(k_h[slots[live]], rk[live], 1e-2 if k_s == "bf16" else 1e-4, "indexer key")
        assert np.all(k_h[untouched] == 7.0)
    _rows_close(_host(w), rw, 1e-2 if w_s == "bf16" else 1e-4, "head weights")


QUERY_CASES = {
    # one query per sequence of the 32-sequence decode batch, V3.2 widths
    "decode_bf16": (32, 1536, "bf16", 11),
    "decode_fp8": (32, 1536, "fp8", 12),
    # enough tokens for the tiled kernel (E4M3 codes and the head's scale
    # written by its epilogue), a partial last 128-token tile
    "tokens_600_fp8": (600, 1536, "fp8", 13),
    # the tiled kernel writing bf16 / fp32 rows itself
    "tokens_600_bf16": (600, 1536, "bf16", 15),
    "tokens_520_f32": (520, 1536, "f32", 16),
    "tokens_7_f32": (7, 1536, "f32", 14),
}


@pytest.mark.parametrize("case", sorted(QUERY_CASES))
def test_indexer_query(dsa, case):
    N, Dq, q_s, seed = QUERY_CASES[case]
    print(f"[indexer_query] {case}: N={N} Dq={Dq} q={q_s}", flush=True)
    torch = U.torch()
    rng = np.random.default_rng(seed)
    cq = g.f32_to_bf16_bits(rng.standard_normal((N, Dq)).astype(np.float32))
    wq = g.f32_to_bf16_bits((rng.standard_normal((8192, Dq)) / math.sqrt(Dq)).astype(np.float32))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).cuda().view(torch.bfloat16)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[q_s]
    q, q_sf = dsa.dsa_indexer_query(t(cq), t(wq), q_dtype=dt)
    torch.cuda.synchronize()
    ref = oracle.indexer_query(cq, wq).reshape(N * 64, 128)
    if q_s == "fp8":
        _check_fp8(q.cpu().numpy().reshape(N * 64, 128), q_sf.cpu().numpy().reshape(N * 64), ref)
    else:
        _rows_close(_host(q).reshape(N * 64, 128), ref, 1e-2 if q_s == "bf16" else 1e-4, "indexer query")


def _gpu_bf16(gen, shape, scale=1.0):
    torch = U.torch()
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)


def _bits(t):
    torch = U.torch()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _sampled(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 10)]))


def test_cache_fill_prefill_16384_sampled(dsa):
    """The prefill size bench.py times (16384 tokens, hidden 7168, fp8 keys):
    inputs drawn on the GPU from a seeded generator, sampled tokens checked
    against the oracle."""
    torch = U.torch()
    N, D = 16384, 7168
    print(f"[cache_fill] prefill_16384_sampled: N={N} D={D}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(61)
    x = _gpu_bf16(gen, (N, D))
    W = _gpu_bf16(gen, (768, D), 1 / math.sqrt(D))
    kv_gamma = 1 + 0.1 * torch.randn(512, generator=gen, device="cuda")
    k_gamma = 1 + 0.1 * torch.randn(128, generator=gen, device="cuda")
    k_beta = 0.1 * torch.randn(128, generator=gen, device="cuda")
    ang = (torch.rand((N, 32), generator=gen, device="cuda") * 2 - 1) * math.pi
    cos, sin = torch.cos(ang), torch.sin(ang)
    slots = torch.arange(N, dtype=torch.int64, device="cuda")
    kv_cache = torch.empty((N, 576), dtype=torch.bfloat16, device="cuda")
    k_cache = torch.empty((N, 128), dtype=torch.uint8, device="cuda")
    k_sf = torch.empty((N,), dtype=torch.uint8, device="cuda")
    w = dsa.dsa_cache_fill(x, W, kv_gamma, k_gamma, k_beta, cos, sin, slots, kv_cache, k_cache, k_sf,
                           w_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = torch.as_tensor(_sampled(N, 61), device="cuda")
    rkv, rk, rw = oracle.cache_fill(_bits(x[rows]), _bits(W), kv_gamma.cpu().numpy(), k_gamma.cpu().numpy(),
                                    k_beta.cpu().numpy(), cos[rows].cpu().numpy(), sin[rows].cpu().numpy())
    kv_h = _host(kv_cache[rows])
    _rows_close(kv_h[:, :512], rkv[:, :512], 1e-2, "normalised latent")
    _rows_close(kv_h[:, 512:], rkv[:, 512:], 1e-2, "rotated key")
    _check_fp8(k_cache[rows].cpu().numpy(), k_sf[rows].cpu().numpy(), rk)
    _rows_close(_host(w[rows]), rw, 1e-2, "head weights")


def test_indexer_query_prefill_16384_sampled(dsa):
    """The prefill size bench.py times (16384 tokens, E4M3 output written by
    the tiled kernel's epilogue): sampled tokens against the oracle."""
    torch = U.torch()
    N, Dq = 16384, 1536
    print(f"[indexer_query] prefill_16384_sampled: N={N} Dq={Dq}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(62)
    cq = _gpu_bf16(gen, (N, Dq))
    wq = _gpu_bf16(gen, (8192, Dq), 1 / math.sqrt(Dq))
    q, q_sf = dsa.dsa_indexer_query(cq, wq, q_dtype=torch.uint8)
    torch.cuda.synchronize()
    rows = torch.as_tensor(_sampled(N, 62), device="cuda")
    n = rows.numel()
    ref = oracle.indexer_query(_bits(cq[rows]), _bits(wq)).reshape(n * 64, 128)
    _check_fp8(q[rows].cpu().numpy().reshape(n * 64, 128), q_sf[rows].cpu().numpy().reshape(n * 64), ref)


@pytest.mark.parametrize("N", [32, 600])
def test_e4m3_scale_floor(dsa, N):
    """Rows whose largest magnitude lies below 448 2^-127: the ue8m0 scale byte
    stops at 0 (2^-127, the smallest scale it holds) instead of wrapping, on
    the GPU as in the oracle.  Cache fill: the indexer key's LayerNorm gain is
    5e-37 (largest key values about 2e-36).  Indexer query: 8 nonzero hidden
    dims per token holding small integers times 2^-62 and weights small
    integers times 2^-62, so every product is a normal fp32 number and every
    query value an exact multiple of 2^-124 below 448 2^-127.  N = 32 takes
    the per-token quantisers, N = 600 the tiled projection's epilogue
    (indexer query)."""
    torch = U.torch()
    print(f"[e4m3_scale_floor] N={N}", flush=True)
    d = _draw(N, 256, 31 + N)
    d["k_gamma"] = np.full(128, 5e-37, np.float32)
    d["k_beta"] = np.zeros(128, np.float32)
    slots = np.arange(N, dtype=np.int64)
    _, k_c, k_sf, _ = _run(dsa, d, slots, N, torch.bfloat16, "fp8", torch.bfloat16)
    _, rk, _ = oracle.cache_fill(d["x"], d["W"], d["kv_gamma"], d["k_gamma"], d["k_beta"],
                                 d["cos"], d["sin"])
    assert np.abs(rk).max() < 448.0 * 2.0 ** -127
    sb = k_sf.cpu().numpy()
    assert np.all(sb == 0), f"scale bytes {np.unique(sb)}"
    _check_fp8(k_c.cpu().numpy(), sb, rk)
    rng = np.random.default_rng(40 + N)
    cqf = np.zeros((N, 1536), np.float32)
    cqf[:, :8] = rng.integers(-2, 3, (N, 8)) * 2.0 ** -62
    wqf = (rng.integers(-3, 4, (8192, 1536)) * 2.0 ** -62).astype(np.float32)
    cq, wq = g.f32_to_bf16_bits(cqf), g.f32_to_bf16_bits(wqf)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).cuda().view(torch.bfloat16)
    q, q_sf = dsa.dsa_indexer_query(t(cq), t(wq), q_dtype=torch.uint8)
    torch.cuda.synchronize()
    ref = oracle.indexer_query(cq, wq).reshape(N * 64, 128)
    assert np.abs(ref).max() < 448.0 * 2.0 ** -127
    qsf = q_sf.cpu().numpy().reshape(N * 64)
    ref_codes, ref_sb = oracle.quantize_e4m3(ref)
    nz = np.abs(ref).max(axis=1) > 0                     # all-zero rows keep scale byte 127
    assert np.all(ref_sb[nz, 0] == 0) and np.array_equal(qsf, ref_sb[:, 0])
    assert np.array_equal(q.cpu().numpy().reshape(N * 64, 128), ref_codes)

"""GPU parity of the absorption products either side of the sparse attention
(dsa_absorb_prepare, dsa_absorb_query, dsa_absorb_output,
dsa_output_projection) against the oracle (fp64).  Small cases come from
numpy draws and are compared whole; the full decode and prefill sizes draw
their inputs on the GPU from a seeded torch generator and compare sampled
tokens (every head and output of each).  bf16 outputs: each row within 1e-2
of its largest value (one bf16 rounding is 2^-9 relative); fp32 outputs:
within 1e-4."""
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


def _bits(t):
    """bf16 tensor -> uint16 bit patterns on the host."""
    torch = U.torch()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _val(t):
    torch = U.torch()
    if t.dtype == torch.bfloat16:
        return g.bf16_bits_to_f32(_bits(t)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _rows_close(got, ref, rtol, what):
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max(axis=1)
    lim = rtol * np.abs(ref).max(axis=1)
    bad = np.nonzero(err > lim)[0]
    assert bad.size == 0, f"{what}: rows {bad[:5]} off by {err[bad[:5]]} (allowed {lim[bad[:5]]})"


def _randn_bf16(gen, shape, scale=1.0):
    torch = U.torch()
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)


def _inputs(N, H, seed, full):
    """qb [N, H, 192], kv_b [H 256, 512], cos / sin [N, 32], o_lat [N, H, 512]
    as GPU tensors: numpy draws (small cases) or a seeded GPU generator."""
    torch = U.torch()
    if full:
        gen = torch.Generator(device="cuda").manual_seed(seed)
        qb = _randn_bf16(gen, (N, H, 192))
        kvb = _randn_bf16(gen, (H * 256, 512), 1 / math.sqrt(512))
        ang = (torch.rand((N, 32), generator=gen, device="cuda") * 2 - 1) * math.pi
        o_lat = _randn_bf16(gen, (N, H, 512), 0.1)
        return qb, kvb, torch.cos(ang), torch.sin(ang), o_lat
    rng = np.random.default_rng(seed)
    bf = lambda a: U.to_dev(g.f32_to_bf16_bits(a.astype(np.float32)), "bf16")
    qb = bf(rng.standard_normal((N, H, 192)))
    kvb = bf(rng.standard_normal((H * 256, 512)) / math.sqrt(512))
    ang = rng.uniform(-math.pi, math.pi, (N, 32))
    o_lat = bf(0.1 * rng.standard_normal((N, H, 512)))
    return (qb, kvb, U.to_dev(np.cos(ang), "f32"), U.to_dev(np.sin(ang), "f32"), o_lat)


def _sample(N, full, seed):
    if not full:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 6)]))


ABSORB_CASES = {
    # decode step of the 32-sequence batch, all 128 heads
    "decode_bf16": (32, 128, "bf16", 41, False),
    "decode_f32": (32, 128, "f32", 42, False),
    # a few heads (a shard): the few-token kernel; ragged token counts
    "heads4_tokens5": (5, 4, "bf16", 43, False),
    "heads4_tokens70_f32": (70, 4, "f32", 44, False),
    # many tokens, a partial last 128-token tile
    "tokens_300": (300, 128, "bf16", 45, False),
    # the prefill (16384 tokens, 128 heads): sampled tokens
    "prefill_16384": (16384, 128, "bf16", 46, True),
}


@pytest.mark.parametrize("case", sorted(ABSORB_CASES))
def test_absorb_query_and_output(dsa, case):
    N, H, dt, seed, full = ABSORB_CASES[case]
    print(f"[absorb] {case}: N={N} H={H} out={dt}", flush=True)
    torch = U.torch()
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[dt]
    qb, kvb, cos, sin, o_lat = _inputs(N, H, seed, full)
    wuk = dsa.dsa_absorb_prepare(kvb)
    q = dsa.dsa_absorb_query(qb, wuk, cos, sin, q_dtype=odt)
    out = dsa.dsa_absorb_output(o_lat, kvb, out_dtype=odt)
    torch.cuda.synchronize()
    kv_np = _val(kvb)
    # the prepared W_UK is a transpose: bit-exact
    wuk_ref = _bits(kvb).reshape(H, 256, 512)[:, :128, :].transpose(0, 2, 1)
    assert np.array_equal(_bits(wuk), wuk_ref), "W_UK transpose"
    rows = torch.as_tensor(_sample(N, full, seed), device="cuda")
    rq = oracle.absorb_query(_val(qb[rows]), kv_np, cos[rows].double().cpu().numpy(),
                             sin[rows].double().cpu().numpy())
    rtol = 1e-2 if dt == "bf16" else 1e-4
    got_q = _val(q[rows])
    _rows_close(got_q[..., :512], rq[..., :512], rtol, "absorbed latent query")
    _rows_close(got_q[..., 512:], rq[..., 512:], rtol, "rotated query")
    ro = oracle.absorb_output(_val(o_lat[rows]), kv_np)
    _rows_close(_val(out[rows]).reshape(len(rows), H, 128), ro.reshape(len(rows), H, 128), rtol,
                "head outputs")


WO_CASES = {
    # decode: 32 tokens, the model's 16384 -> 7168 (split reduction + finish)
    "decode_bf16": (32, 16384, 7168, "bf16", 51, False),
    "decode_f32": (32, 16384, 7168, "f32", 52, False),
    "tokens_300_small": (300, 1024, 256, "f32", 53, False),
    # many tokens: the tiled kernel, a partial last tile
    "tokens_2100": (2100, 1024, 7168, "bf16", 54, False),
    # 256-token tiles (long reduction, enough workgroups), a partial last tile
    "tokens_2400_wide": (2400, 1024, 7168, "bf16", 56, False),
    "tokens_2400_wide_f32": (2400, 1024, 7168, "f32", 57, False),
    # the prefill: 16384 tokens, sampled
    "prefill_16384": (16384, 16384, 7168, "bf16", 55, True),
}


@pytest.mark.parametrize("case", sorted(WO_CASES))
def test_output_projection(dsa, case):
    N, Din, Dout, dt, seed, full = WO_CASES[case]
    print(f"[wo] {case}: N={N} Din={Din} Dout={Dout} out={dt}", flush=True)
    torch = U.torch()
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[dt]
    if full:
        gen = torch.Generator(device="cuda").manual_seed(seed)
        x = _randn_bf16(gen, (N, Din))
        W = _randn_bf16(gen, (Dout, Din), 1 / math.sqrt(Din))
    else:
        rng = np.random.default_rng(seed)
        x = U.to_dev(g.f32_to_bf16_bits(rng.standard_normal((N, Din)).astype(np.float32)), "bf16")
        W = U.to_dev(g.f32_to_bf16_bits((rng.standard_normal((Dout, Din)) / math.sqrt(Din)).astype(np.float32)), "bf16")
    out = dsa.dsa_output_projection(x, W, out_dtype=odt)
    torch.cuda.synchronize()
    rows = torch.as_tensor(_sample(N, full, seed), device="cuda")
    ref = oracle.linear_bf16(_bits(x[rows]), _bits(W))
    _rows_close(_val(out[rows]), ref, 1e-2 if dt == "bf16" else 1e-4, "output projection")


def test_minimum_and_empty_sizes(dsa):
    """One token and one head through every absorption entry point, the
    smallest output projection (64 -> 128), and zero tokens (nothing launched,
    empty outputs)."""
    torch = U.torch()
    print("[absorb] minimum and empty sizes", flush=True)
    qb, kvb, cos, sin, o_lat = _inputs(1, 1, 71, False)
    wuk = dsa.dsa_absorb_prepare(kvb)
    q = dsa.dsa_absorb_query(qb, wuk, cos, sin, q_dtype=torch.float32)
    out = dsa.dsa_absorb_output(o_lat, kvb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kv_np = _val(kvb)
    rq = oracle.absorb_query(_val(qb), kv_np, cos.double().cpu().numpy(), sin.double().cpu().numpy())
    _rows_close(_val(q)[..., :512], rq[..., :512], 1e-4, "absorbed latent query")
    _rows_close(_val(q)[..., 512:], rq[..., 512:], 1e-4, "rotated query")
    _rows_close(_val(out).reshape(1, 1, 128), oracle.absorb_output(_val(o_lat), kv_np).reshape(1, 1, 128),
                1e-4, "head outputs")
    rng = np.random.default_rng(72)
    x = U.to_dev(g.f32_to_bf16_bits(rng.standard_normal((1, 64)).astype(np.float32)), "bf16")
    W = U.to_dev(g.f32_to_bf16_bits(rng.standard_normal((128, 64)).astype(np.float32)), "bf16")
    y = dsa.dsa_output_projection(x, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _rows_close(_val(y), oracle.linear_bf16(_bits(x), _bits(W)), 1e-4, "output projection")
    # zero tokens: empty results, no launch
    e_qb, e_o = qb[:0], o_lat[:0]
    assert dsa.dsa_absorb_query(e_qb, wuk, cos[:0], sin[:0]).shape == (0, 1, 576)
    assert dsa.dsa_absorb_output(e_o, kvb).shape == (0, 128)
    assert dsa.dsa_output_projection(x[:0], W).shape == (0, 128)
    torch.cuda.synchronize()

"""The -DDSA_DEBUG build of libdsa on the GPU (MI355X only).

The debug build fills every kernel's LDS with 0xff bytes before first use and
checks index rows on the device: the top-K output (entries in [-1, S), valid
entries strictly ascending, -1 padding last) and the rows the attention reads
(entries in [-1, S)).  Here:
  * the whole path through the debug build still matches the oracle (so no
    kernel reads LDS it did not write, and the top-K rows pass the check);
  * rows with entries outside [-1, S), which the release build skips, are
    rejected by the debug build with DSA_ERR_INVALID_ARG.
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


@pytest.fixture
def debug_build(dsa):
    """Routes the binding to libdsa_debug.so for one test."""
    from sparse_latent_attention_lightning_amd import _binding as B
    from sparse_latent_attention_lightning_amd import build as Bld
    saved = B.lib()
    B._lib = B.load_library(Bld.DEBUG_LIB)  # fails loudly if it was not built
    try:
        yield dsa
    finally:
        B._lib = saved


def _forward_check(dsa, cfg):
    x = U.upload_all(cfg)
    o, lse, idx = dsa.dsa_forward(U.shape_of(cfg), x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                  x["q_sf"], x["k_sf"])
    U.torch().cuda.synchronize()
    rows = cfg.B * cfg.T
    rb = np.repeat(np.arange(cfg.B, dtype=np.int32), cfg.T)
    rt = np.tile(np.arange(cfg.T, dtype=np.int32), cfg.B)
    qi = g.full(cfg, "q_idx")
    k = g.full(cfg, "k_idx")
    w = g.full(cfg, "w").reshape(rows, cfg.HI)
    if cfg.idx_dtype == "fp8":
        sc = oracle.indexer_scores(cfg, rb, rt, qi[0].reshape(rows, cfg.HI, cfg.DI), w, k[0],
                                   qi[1].reshape(rows, cfg.HI, -1), k[1])
    else:
        sc = oracle.indexer_scores(cfg, rb, rt, qi.reshape(rows, cfg.HI, cfg.DI), w, k)
    ref_idx = oracle.topk(cfg, sc)
    assert np.array_equal(idx.cpu().numpy().reshape(rows, -1), ref_idx), f"{cfg.name}: selection"
    ro, rl = oracle.sparse_mla(cfg, rb, g.full(cfg, "q").reshape(rows, cfg.H, cfg.D), g.full(cfg, "kv"), ref_idx)
    got = U.dev_to_np(o, cfg.mla_dtype).reshape(rows, cfg.H, cfg.Dc)
    if cfg.mla_dtype == "bf16":
        got = g.bf16_bits_to_f32(got)
    U.assert_rows_close(got, ro, U.RTOL[cfg.mla_dtype], what=f"debug build {cfg.name} o")


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("decode_8k", dict(B=2, S=4096, integer=True)),                  # split attention + combine
    ("decode_64k_fp8", dict(B=2, S=4096, integer=True)),             # e4m3 streaming indexer
    ("prefill_16k", dict(T=40, S=2500, integer=True)),               # prefill indexer, no splits
    ("decode_128k", dict(B=1, S=40000, cluster=0, integer=True)),    # two-stage top-K
    ("decode_128k", dict(B=1, S=40000, K=20000, cluster=0, integer=True)),  # long-row top-K
])
def test_debug_build_path_matches_oracle(debug_build, name, over):
    _forward_check(debug_build, g.CONFIGS[name].replace(**over))


def test_debug_build_rejects_out_of_range_entries(dsa, debug_build):
    torch = U.torch()
    cfg = g.CONFIGS["decode_8k"].replace(B=2, S=4096, K=512)
    x = U.upload_all(cfg)
    rng = np.random.default_rng(3)
    idx = np.stack([np.sort(rng.choice(cfg.S, cfg.K_eff, replace=False)) for _ in range(cfg.B)]).astype(np.int32)
    for bad in (cfg.S, -2):
        wrong = idx.copy()
        wrong[1, 7] = bad
        d_idx = torch.from_numpy(wrong.reshape(cfg.B, 1, -1)).cuda()
        with pytest.raises(dsa.DsaError, match="debug check of attention index rows"):
            debug_build.dsa_sparse_mla_fwd(U.shape_of(cfg), x["q"], x["kv"], d_idx)
    # valid rows (and -1 anywhere) pass the check
    ok = idx.copy()
    ok[0, ::3] = -1
    o, _ = debug_build.dsa_sparse_mla_fwd(U.shape_of(cfg), x["q"], x["kv"], torch.from_numpy(ok.reshape(cfg.B, 1, -1)).cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()

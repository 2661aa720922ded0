"""dsa_forward_noalloc (the whole path on the library's own scratch, for
callers that cannot allocate) against dsa_forward on a caller workspace:
two calls in a row, the second with a smaller input, each compared with
dsa_forward on the same inputs at the parity bar (the selection exactly, o
per (b, t, h) row within 2e-2 of its largest value, lse likewise; the two
share every kernel, so they agree bit for bit in practice).  A shape whose
scratch exceeds the library's 64 MiB is refused before any launch."""
import ctypes

import numpy as np
import pytest

import dsa_inputs as g
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_lightning_amd as m
    m.lib()
    return m


def _compare(dsa, cfg):
    torch = U.torch()
    x = U.upload_all(cfg)
    shape = U.shape_of(cfg)
    args = (shape, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["q_sf"], x["k_sf"])
    o_ref, l_ref, i_ref = dsa.dsa_forward(*args)
    o, l, i = dsa.dsa_forward_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.equal(i, i_ref), f"{cfg.name}: selection differs"
    rows = cfg.B * cfg.T
    a = g.bf16_bits_to_f32(U.dev_to_np(o, "bf16")).reshape(rows, cfg.H, cfg.Dc)
    b = g.bf16_bits_to_f32(U.dev_to_np(o_ref, "bf16")).reshape(rows, cfg.H, cfg.Dc)
    U.assert_rows_close(a, b, U.RTOL["bf16"], what=f"{cfg.name} o")
    ln, lr = l.cpu().numpy(), l_ref.cpu().numpy()
    assert np.all(np.abs(ln - lr) <= U.RTOL["bf16"] * np.maximum(1, np.abs(lr)))
    return torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(l, l_ref)


def test_noalloc_matches_forward_twice_then_smaller(dsa):
    big = g.CONFIGS["decode_8k"].replace(B=16)
    small = g.CONFIGS["decode_64k_fp8"].replace(B=3, S=5000)
    print(f"[noalloc] {big.name} B={big.B} S={big.S}, then {small.name} B={small.B} S={small.S}",
          flush=True)
    same1 = _compare(dsa, big)
    same2 = _compare(dsa, small)
    print(f"[noalloc] bitwise equal to dsa_forward: {same1}, {same2}", flush=True)


def test_noalloc_refuses_oversized_shape(dsa):
    cfg = g.CONFIGS["prefill_16k"].replace(T=4096, S=4096)   # 64 MiB of scores alone
    shape = U.shape_of(cfg)
    assert dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD) > 64 << 20
    L = dsa.lib()
    P = ctypes.c_void_p(256)   # never dereferenced: refused on the host
    rc = L.dsa_forward_noalloc(ctypes.byref(shape), P, None, P, None, P, P, P, None, P, None, None)
    assert rc == 3 and "scratch" in L.dsa_last_error().decode()

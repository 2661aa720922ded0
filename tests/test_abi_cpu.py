"""The C ABI on the host (no GPU needed): the library loads, exports every
entry point include/dsa.h declares, and rejects bad arguments before it
touches the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def dsa():
    import sparse_latent_attention_lightning_amd as m
    if not os.path.exists(m._binding.LIB_PATH):
        from sparse_latent_attention_lightning_amd import build
        build.build()
    m.lib()
    return m


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_forward",
              "dsa_workspace_bytes", "dsa_status_str", "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(dsa._binding.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), f"{n} declared in dsa.h but not exported"


def test_status_strings(dsa):
    L = dsa.lib()
    assert L.dsa_status_str(0) == b"DSA_OK"
    assert L.dsa_status_str(3) == b"DSA_ERR_WORKSPACE"
    assert L.dsa_status_str(99) == b"DSA_ERR_UNKNOWN"


def _v32(dsa, **kw):
    base = dict(B=32, T=1, S=8192, HI=64, DI=128, H=128, Dc=512, Dr=64, K=2048,
                idx_scale=1 / (8 * 128 ** 0.5), sm_scale=192 ** -0.5)
    base.update(kw)
    return dsa.make_shape(**base)


def test_workspace_sizes(dsa):
    s = _v32(dsa)
    topk = dsa.workspace_bytes(s, dsa.ENTRY_TOPK)
    mla = dsa.workspace_bytes(s, dsa.ENTRY_SPARSE_MLA)
    fwd = dsa.workspace_bytes(s, dsa.ENTRY_FORWARD)
    assert topk == 0                               # one workgroup per 8192-key row
    splits = 8                                      # 32 rows x 8 splits fill 256 CUs
    assert mla == 32 * splits * 128 * 512 * 2 + 32 * splits * 128 * 4  # bf16 o and fp32 lse partials
    assert fwd >= 32 * 8192 * 4 + 32 * 2048 * 4 + mla
    long = _v32(dsa, B=8, S=131072)
    assert dsa.workspace_bytes(long, dsa.ENTRY_TOPK) == 8 * 8 * 2048 * 8  # 8 chunks of 16 K keys
    longer = _v32(dsa, B=1, S=300000)  # 19 chunks of 16 K would overflow one merge: 10 of 32 K
    assert dsa.workspace_bytes(longer, dsa.ENTRY_TOPK) == 10 * 2048 * 8
    # candidates that fit no merge (19 chunks of 32 K): the long-row select, per
    # row 4 meeting words, a 4096-bin histogram, one pair count per 4096-key
    # chunk (rounded up to 64 over all rows) and 4096 (key, index) pairs per chunk
    longest = _v32(dsa, B=1, S=600000)  # 147 chunks, the last one ragged
    assert dsa.workspace_bytes(longest, dsa.ENTRY_TOPK) == 32 + 4096 * 4 + 192 * 4 + 147 * 4096 * 8
    prefill = _v32(dsa, B=1, T=16384, S=16384)
    assert dsa.workspace_bytes(prefill, dsa.ENTRY_SPARSE_MLA) == 0         # no splits
    with pytest.raises(dsa.DsaError):
        dsa.workspace_bytes(_v32(dsa, K=0), dsa.ENTRY_TOPK)
    with pytest.raises(dsa.DsaError):
        dsa.workspace_bytes(s, 7)
    # the fused index scores -> top-K: the scores, then per row two state
    # words and a 4096-bin histogram
    it = dsa.workspace_bytes(s, dsa.ENTRY_INDEXER_TOPK)
    assert it == 32 * 8192 * 4 + 32 * (16 + 4096 * 4)
    with pytest.raises(dsa.DsaError):            # prefill: not covered by the fused launch
        dsa.workspace_bytes(prefill, dsa.ENTRY_INDEXER_TOPK)


def test_indexer_topk_rejects_uncovered_shapes_on_host(dsa):
    L = dsa.lib()
    P = ctypes.c_void_p(256)   # never dereferenced: refused on the host
    for bad in (dict(T=8, S=4096), dict(S=300000), dict(HI=32), dict(idx_dtype=0)):
        s = _v32(dsa, **bad)
        rc = L.dsa_indexer_topk(ctypes.byref(s), None, P, None, P, None, P, P, P, 1 << 40, None)
        assert rc == 2, bad
    rc = L.dsa_indexer_topk(ctypes.byref(_v32(dsa)), None, P, None, P, None, P, P, P, 1024, None)
    assert rc == 3 and "workspace" in L.dsa_last_error().decode()


@pytest.mark.parametrize("bad,msg", [
    (dict(B=0), "positive"), (dict(T=9, S=8), "exceeds"), (dict(K=0), "K must"),
    (dict(idx_dtype=2, DI=100), "fp8"), (dict(w_dtype=2), "w_dtype"), (dict(mla_dtype=2), "mla_dtype"),
    (dict(HI=-1), "HI"),
])
def test_bad_shapes_rejected_on_host(dsa, bad, msg):
    L = dsa.lib()
    s = _v32(dsa, **bad)
    P = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    for rc in (L.dsa_indexer_scores(ctypes.byref(s), P, None, P, None, P, P, None),
               L.dsa_topk(ctypes.byref(s), P, P, None, 0, None),
               L.dsa_sparse_mla_fwd(ctypes.byref(s), P, P, P, P, None, None, 0, None),
               L.dsa_forward(ctypes.byref(s), P, None, P, None, P, P, P, None, P, None, None, 0, None)):
        assert rc == 1
        assert msg in L.dsa_last_error().decode()


def test_null_and_misaligned_pointers_rejected(dsa):
    L = dsa.lib()
    s = _v32(dsa)
    P = ctypes.c_void_p(256)
    rc = L.dsa_indexer_scores(ctypes.byref(s), None, None, P, None, P, P, None)
    assert rc == 1 and "q_idx is NULL" in L.dsa_last_error().decode()
    rc = L.dsa_sparse_mla_fwd(ctypes.byref(s), P, ctypes.c_void_p(258), P, P, None, None, 0, None)
    assert rc == 1 and "kv is not 16-byte aligned" in L.dsa_last_error().decode()
    rc = L.dsa_indexer_scores(ctypes.byref(_v32(dsa, idx_dtype=2)), P, None, P, None, P, P, None)
    assert rc == 1 and "q_sf" in L.dsa_last_error().decode()
    rc = L.dsa_topk(None, P, P, None, 0, None)
    assert rc == 1 and "shape is NULL" in L.dsa_last_error().decode()


def test_ragged_entry_points_check_seq_lens_on_host(dsa):
    L = dsa.lib()
    s = _v32(dsa)
    P = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(258)
    rc = L.dsa_indexer_scores_ragged(ctypes.byref(s), odd, P, None, P, None, P, P, None)
    assert rc == 1 and "seq_lens is not 4-byte aligned" in L.dsa_last_error().decode()
    rc = L.dsa_forward_ragged(ctypes.byref(s), odd, P, None, P, None, P, P, P, None, P, None,
                              P, 1 << 40, None)
    assert rc == 1 and "seq_lens is not 4-byte aligned" in L.dsa_last_error().decode()
    rc = L.dsa_indexer_scores_ragged(None, None, P, None, P, None, P, P, None)
    assert rc == 1 and "shape is NULL" in L.dsa_last_error().decode()


def test_forward_workspace_too_small(dsa):
    L = dsa.lib()
    s = _v32(dsa)
    P = ctypes.c_void_p(256)
    rc = L.dsa_forward(ctypes.byref(s), P, None, P, None, P, P, P, None, P, None, P, 1024, None)
    assert rc == 3 and "workspace" in L.dsa_last_error().decode()


@pytest.mark.parametrize("over,msg", [
    (dict(B=65536), "65535 rows"),                 # one grid row per query row in top-K and attention
    (dict(B=1, S=2048 * 4096 + 1), "long-row select's 8388608 keys"),  # the top-K's 2048 chunks of 4096
])
def test_forward_shape_limits_fail_before_any_launch(dsa, over, msg):
    """dsa_forward checks every step's limits before its first launch: without a
    GPU a launch would fail with DSA_ERR_HIP, so DSA_ERR_UNSUPPORTED here means
    nothing was enqueued."""
    L = dsa.lib()
    s = _v32(dsa, **over)
    P = ctypes.c_void_p(256)
    rc = L.dsa_forward(ctypes.byref(s), P, None, P, None, P, P, P, None, P, None, P, 1 << 50, None)
    assert rc == 2 and msg in L.dsa_last_error().decode()


def test_timing_session_on_host(dsa):
    # no launches happen, so no event is created and no device is touched
    with pytest.raises(dsa.DsaError, match="no active session"):
        dsa.dsa_timing_end()
    dsa.dsa_timing_begin()
    with pytest.raises(dsa.DsaError, match="already active"):
        dsa.dsa_timing_begin()
    assert dsa.dsa_timing_end() == {}
    # a launch rejected on the host is not timed and leaves no record
    dsa.dsa_timing_begin()
    L = dsa.lib()
    assert L.dsa_topk(ctypes.byref(_v32(dsa, K=0)), ctypes.c_void_p(256), ctypes.c_void_p(256), None, 0, None) == 1
    assert dsa.dsa_timing_end() == {}


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import sparse_latent_attention_lightning_amd._binding as b
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(ImportError):
        b.lib()


def test_absorption_entry_points_check_arguments_on_host(dsa):
    L = dsa.lib()
    P = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert L.dsa_absorb_prepare(-1, P, P, None) == 1
    assert L.dsa_absorb_prepare(4, None, P, None) == 1
    assert L.dsa_absorb_prepare(0, None, None, None) == 0          # nothing to do
    assert L.dsa_absorb_query(32, 128, P, P, P, P, 2, P, None) == 2  # no E4M3 query
    assert L.dsa_absorb_query(-1, 128, P, P, P, P, 1, P, None) == 1
    assert L.dsa_absorb_query(32, 128, P, P, None, P, 1, P, None) == 1
    assert L.dsa_absorb_query(0, 128, None, None, None, None, 1, None, None) == 0
    assert L.dsa_absorb_output(32, 128, P, P, 2, P, None) == 2
    assert L.dsa_absorb_output(32, 128, P, None, 1, P, None) == 1
    assert L.dsa_output_projection(32, 100, 7168, P, P, 1, P, None, 0, None) == 1  # Din % 64
    assert "Din" in L.dsa_last_error().decode()
    assert L.dsa_output_projection(32, 16384, 7000, P, P, 1, P, None, 0, None) == 1  # Dout % 128
    assert L.dsa_output_projection(32, 16384, 7168, P, P, 2, P, None, 0, None) == 2
    # few tokens split the 16384-wide reduction into 16 slices of fp32 partials
    assert L.dsa_output_projection_workspace_bytes(32, 16384, 7168) == 16 * 32 * 7168 * 4
    assert L.dsa_output_projection_workspace_bytes(16384, 16384, 7168) == 0  # tiled: none
    assert L.dsa_output_projection_workspace_bytes(32, 100, 7168) == ctypes.c_size_t(-1).value

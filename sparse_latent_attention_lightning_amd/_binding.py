"""ctypes binding of libdsa (include/dsa.h), same entry-point names.

Argument marshalling only: shape checks, output/workspace allocation with
torch, device pointers and the current HIP stream go to the C ABI; every step
of the computation runs in the library's HIP kernels.  There is no fallback:
if libdsa.so is missing or fails to load, the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
ENTRY_TOPK, ENTRY_SPARSE_MLA, ENTRY_FORWARD, ENTRY_INDEXER_TOPK = 0, 1, 2, 3
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
          3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}

_ELEM = {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16}


class DsaShape(ctypes.Structure):
    """Mirror of dsa_shape_t."""
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "S", "HI", "DI", "H", "Dc", "Dr", "K")] + [
        ("idx_scale", ctypes.c_float), ("sm_scale", ctypes.c_float),
        ("idx_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("mla_dtype", ctypes.c_int32)]

    @property
    def K_eff(self) -> int:
        return min(self.K, self.S)

    def __repr__(self) -> str:
        return "DsaShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class DsaKernelTime(ctypes.Structure):
    """Mirror of dsa_kernel_time_t."""
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("dropped", ctypes.c_int32), ("total_ms", ctypes.c_double),
                ("min_ms", ctypes.c_double), ("max_ms", ctypes.c_double)]


class DsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def make_shape(B, T, S, HI, DI, H, Dc, Dr, K, idx_scale, sm_scale,
               idx_dtype=DSA_BF16, w_dtype=DSA_BF16, mla_dtype=DSA_BF16) -> DsaShape:
    return DsaShape(B, T, S, HI, DI, H, Dc, Dr, K, idx_scale, sm_scale, idx_dtype, w_dtype,
                    mla_dtype)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdsa (raises if it is not built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Loads a build of libdsa at `path` (the release build, or the
    -DDSA_DEBUG one) and declares its entry points."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run "
                          "`python -m sparse_latent_attention_lightning_amd.build`")
    L = ctypes.CDLL(path)
    P, sz = ctypes.c_void_p, ctypes.c_size_t
    sp = ctypes.POINTER(DsaShape)
    L.dsa_indexer_scores.argtypes = [sp, P, P, P, P, P, P, P]
    L.dsa_indexer_scores_ragged.argtypes = [sp, P, P, P, P, P, P, P, P]
    L.dsa_topk.argtypes = [sp, P, P, P, sz, P]
    L.dsa_sparse_mla_fwd.argtypes = [sp, P, P, P, P, P, P, sz, P]
    L.dsa_forward.argtypes = [sp, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    L.dsa_forward_ragged.argtypes = [sp, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    L.dsa_forward_noalloc.argtypes = [sp, P, P, P, P, P, P, P, P, P, P, P]
    L.dsa_indexer_topk.argtypes = [sp, P, P, P, P, P, P, P, P, sz, P]
    i32 = ctypes.c_int32
    L.dsa_cache_fill.argtypes = [i32, i32] + [P] * 8 + [i32, P, i32, P, P, i32, P, P, sz, P]
    L.dsa_cache_fill.restype = ctypes.c_int
    L.dsa_cache_fill_workspace_bytes.argtypes = [i32, i32]
    L.dsa_cache_fill_workspace_bytes.restype = sz
    L.dsa_indexer_query.argtypes = [i32, i32, P, P, i32, P, P, P, sz, P]
    L.dsa_indexer_query.restype = ctypes.c_int
    L.dsa_indexer_query_workspace_bytes.argtypes = [i32, i32]
    L.dsa_indexer_query_workspace_bytes.restype = sz
    L.dsa_absorb_prepare.argtypes = [i32, P, P, P]
    L.dsa_absorb_query.argtypes = [i32, i32, P, P, P, P, i32, P, P]
    L.dsa_absorb_output.argtypes = [i32, i32, P, P, i32, P, P]
    L.dsa_output_projection.argtypes = [i32, i32, i32, P, P, i32, P, P, sz, P]
    for f in ("dsa_absorb_prepare", "dsa_absorb_query", "dsa_absorb_output",
              "dsa_output_projection"):
        getattr(L, f).restype = ctypes.c_int
    L.dsa_output_projection_workspace_bytes.argtypes = [i32, i32, i32]
    L.dsa_output_projection_workspace_bytes.restype = sz
    for f in ("dsa_indexer_scores", "dsa_indexer_scores_ragged", "dsa_topk",
              "dsa_sparse_mla_fwd", "dsa_forward", "dsa_forward_ragged", "dsa_forward_noalloc",
              "dsa_indexer_topk"):
        getattr(L, f).restype = ctypes.c_int
    L.dsa_workspace_bytes.argtypes = [sp, ctypes.c_int32]
    L.dsa_workspace_bytes.restype = ctypes.c_size_t
    L.dsa_timing_begin.argtypes = []
    L.dsa_timing_begin.restype = ctypes.c_int
    L.dsa_timing_end.argtypes = [ctypes.POINTER(DsaKernelTime), ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_int32)]
    L.dsa_timing_end.restype = ctypes.c_int
    L.dsa_status_str.argtypes = [ctypes.c_int]
    L.dsa_status_str.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_last_error.restype = ctypes.c_char_p
    return L


def _check(status: int):
    if status != 0:
        raise DsaError(status, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _req(t: torch.Tensor, name: str, shape: Tuple[int, ...], dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ws_bytes(ws: Optional[torch.Tensor], device) -> int:
    """Byte size of a caller workspace: a contiguous uint8 GPU tensor on
    `device` (None: no workspace)."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError("ws must be a tensor")
    if ws.device != device:
        raise ValueError(f"ws is on {ws.device}, expected {device}")
    if ws.dtype != torch.uint8:
        raise ValueError(f"ws has dtype {ws.dtype}, expected torch.uint8")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    return ws.numel()


def _idx_dtypes(code):
    if code == DSA_FP8_E4M3:
        return (torch.uint8, torch.float8_e4m3fn)
    return (_ELEM[code],)


def workspace_bytes(shape: DsaShape, entry: int) -> int:
    n = lib().dsa_workspace_bytes(ctypes.byref(shape), entry)
    if n == ctypes.c_size_t(-1).value:
        raise DsaError(1, lib().dsa_last_error().decode())
    return n


def _workspace(shape: DsaShape, entry: int, device) -> Optional[torch.Tensor]:
    n = workspace_bytes(shape, entry)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf):
    s = shape
    dev = q_idx.device
    _req(q_idx, "q_idx", (s.B, s.T, s.HI, s.DI), _idx_dtypes(s.idx_dtype))
    _req(k_idx, "k_idx", (s.B, s.S, s.DI), _idx_dtypes(s.idx_dtype), dev)
    _req(w, "w", (s.B, s.T, s.HI), (_ELEM[s.w_dtype],), dev)
    if s.idx_dtype == DSA_FP8_E4M3:
        _req(q_sf, "q_sf", (s.B, s.T, s.HI, s.DI // 128), (torch.uint8,), dev)
        _req(k_sf, "k_sf", (s.B, s.S, s.DI // 128), (torch.uint8,), dev)
    return dev


def _check_mla(shape, q, kv, idx):
    s = shape
    dev = q.device
    _req(q, "q", (s.B, s.T, s.H, s.Dc + s.Dr), (_ELEM[s.mla_dtype],))
    _req(kv, "kv", (s.B, s.S, s.Dc + s.Dr), (_ELEM[s.mla_dtype],), dev)
    if idx is not None:
        _req(idx, "idx", (s.B, s.T, s.K_eff), (torch.int32,), dev)
    return dev


def _seq_lens(shape: DsaShape, seq_lens, dev):
    _req(seq_lens, "seq_lens", (shape.B,), (torch.int32,), dev)
    return seq_lens


def dsa_indexer_scores(shape: DsaShape, q_idx, k_idx, w, q_sf=None, k_sf=None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores [B, T, S] fp32 (future keys -inf)."""
    dev = _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.S), dtype=torch.float32, device=dev)
    _req(out, "scores", (shape.B, shape.T, shape.S), (torch.float32,), dev)
    _check(lib().dsa_indexer_scores(ctypes.byref(shape), _ptr(q_idx), _ptr(q_sf), _ptr(k_idx),
                                    _ptr(k_sf), _ptr(w), _ptr(out), _stream(dev)))
    return out


def dsa_indexer_scores_ragged(shape: DsaShape, seq_lens, q_idx, k_idx, w, q_sf=None, k_sf=None,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores [B, T, S] fp32 of a ragged batch: sequence b holds
    seq_lens[b] keys (int32 [B] on the device) and its queries are its last T
    positions."""
    dev = _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf)
    _seq_lens(shape, seq_lens, dev)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.S), dtype=torch.float32, device=dev)
    _req(out, "scores", (shape.B, shape.T, shape.S), (torch.float32,), dev)
    _check(lib().dsa_indexer_scores_ragged(ctypes.byref(shape), _ptr(seq_lens), _ptr(q_idx),
                                           _ptr(q_sf), _ptr(k_idx), _ptr(k_sf), _ptr(w), _ptr(out),
                                           _stream(dev)))
    return out


def dsa_indexer_topk(shape: DsaShape, q_idx, k_idx, w, q_sf=None, k_sf=None, seq_lens=None,
                     out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Index scores and top-K in one launch (decode shapes): idx [B, T, K_eff]
    int32, exactly dsa_topk of dsa_indexer_scores.  The row scores remain at
    the start of ws ([B, T, S] fp32)."""
    dev = _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf)
    if seq_lens is not None:
        _seq_lens(shape, seq_lens, dev)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.K_eff), dtype=torch.int32, device=dev)
    _req(out, "idx", (shape.B, shape.T, shape.K_eff), (torch.int32,), dev)
    if ws is None:
        ws = _workspace(shape, ENTRY_INDEXER_TOPK, dev)
    _check(lib().dsa_indexer_topk(ctypes.byref(shape), _ptr(seq_lens), _ptr(q_idx), _ptr(q_sf),
                                  _ptr(k_idx), _ptr(k_sf), _ptr(w), _ptr(out), _ptr(ws),
                                  _ws_bytes(ws, dev), _stream(dev)))
    return out


def dsa_topk(shape: DsaShape, scores, out: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-K index rows [B, T, min(K, S)] int32, ascending, -1 padded."""
    _req(scores, "scores", (shape.B, shape.T, shape.S), (torch.float32,))
    dev = scores.device
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.K_eff), dtype=torch.int32, device=dev)
    _req(out, "idx", (shape.B, shape.T, shape.K_eff), (torch.int32,), dev)
    if ws is None:
        ws = _workspace(shape, ENTRY_TOPK, dev)
    _check(lib().dsa_topk(ctypes.byref(shape), _ptr(scores), _ptr(out), _ptr(ws),
                          _ws_bytes(ws, dev), _stream(dev)))
    return out


def dsa_sparse_mla_fwd(shape: DsaShape, q, kv, idx, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                       ws: Optional[torch.Tensor] = None):
    """Absorbed sparse latent attention: (o [B,T,H,Dc], lse [B,T,H] fp32 or None)."""
    dev = _check_mla(shape, q, kv, idx)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.H, shape.Dc), dtype=q.dtype, device=dev)
    _req(out, "o", (shape.B, shape.T, shape.H, shape.Dc), (q.dtype,), dev)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.T, shape.H), dtype=torch.float32, device=dev)
    if lse is not None:
        _req(lse, "lse", (shape.B, shape.T, shape.H), (torch.float32,), dev)
    if ws is None:
        ws = _workspace(shape, ENTRY_SPARSE_MLA, dev)
    _check(lib().dsa_sparse_mla_fwd(ctypes.byref(shape), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out),
                                    _ptr(lse), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)))
    return out, lse


def dsa_forward(shape: DsaShape, q_idx, k_idx, w, q, kv, q_sf=None, k_sf=None,
                want_idx: bool = True, want_lse: bool = True, ws: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None):
    """The whole hot path: (o, lse or None, idx or None)."""
    return dsa_forward_ragged(shape, None, q_idx, k_idx, w, q, kv, q_sf, k_sf, want_idx, want_lse,
                              ws, out, idx_out, lse)


def dsa_forward_ragged(shape: DsaShape, seq_lens, q_idx, k_idx, w, q, kv, q_sf=None, k_sf=None,
                       want_idx: bool = True, want_lse: bool = True,
                       ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       idx_out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """The whole hot path over a ragged batch (seq_lens int32 [B] on the
    device, or None for full sequences): (o, lse or None, idx or None)."""
    dev = _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf)
    if seq_lens is not None:
        _seq_lens(shape, seq_lens, dev)
    _check_mla(shape, q, kv, None)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.H, shape.Dc), dtype=q.dtype, device=dev)
    _req(out, "o", (shape.B, shape.T, shape.H, shape.Dc), (q.dtype,), dev)
    if idx_out is None and want_idx:
        idx_out = torch.empty((shape.B, shape.T, shape.K_eff), dtype=torch.int32, device=dev)
    if idx_out is not None:
        _req(idx_out, "idx_out", (shape.B, shape.T, shape.K_eff), (torch.int32,), dev)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.T, shape.H), dtype=torch.float32, device=dev)
    if lse is not None:
        _req(lse, "lse", (shape.B, shape.T, shape.H), (torch.float32,), dev)
    if ws is None:
        ws = _workspace(shape, ENTRY_FORWARD, dev)
    nws = _ws_bytes(ws, dev)
    if seq_lens is None:
        _check(lib().dsa_forward(ctypes.byref(shape), _ptr(q_idx), _ptr(q_sf), _ptr(k_idx),
                                 _ptr(k_sf), _ptr(w), _ptr(q), _ptr(kv), _ptr(idx_out), _ptr(out),
                                 _ptr(lse), _ptr(ws), nws, _stream(dev)))
    else:
        _check(lib().dsa_forward_ragged(ctypes.byref(shape), _ptr(seq_lens), _ptr(q_idx),
                                        _ptr(q_sf), _ptr(k_idx), _ptr(k_sf), _ptr(w), _ptr(q),
                                        _ptr(kv), _ptr(idx_out), _ptr(out), _ptr(lse), _ptr(ws),
                                        nws, _stream(dev)))
    return out, lse, idx_out


def dsa_forward_noalloc(shape: DsaShape, q_idx, k_idx, w, q, kv, q_sf=None, k_sf=None,
                        want_idx: bool = True, want_lse: bool = True,
                        out: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None):
    """The whole hot path on the library's own scratch (no workspace; the C
    call allocates nothing): (o, lse or None, idx or None).  Outputs not
    given are allocated here, before the call."""
    dev = _check_indexer(shape, q_idx, k_idx, w, q_sf, k_sf)
    _check_mla(shape, q, kv, None)
    if out is None:
        out = torch.empty((shape.B, shape.T, shape.H, shape.Dc), dtype=q.dtype, device=dev)
    _req(out, "o", (shape.B, shape.T, shape.H, shape.Dc), (q.dtype,), dev)
    if idx_out is None and want_idx:
        idx_out = torch.empty((shape.B, shape.T, shape.K_eff), dtype=torch.int32, device=dev)
    if idx_out is not None:
        _req(idx_out, "idx_out", (shape.B, shape.T, shape.K_eff), (torch.int32,), dev)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.T, shape.H), dtype=torch.float32, device=dev)
    if lse is not None:
        _req(lse, "lse", (shape.B, shape.T, shape.H), (torch.float32,), dev)
    _check(lib().dsa_forward_noalloc(ctypes.byref(shape), _ptr(q_idx), _ptr(q_sf), _ptr(k_idx),
                                     _ptr(k_sf), _ptr(w), _ptr(q), _ptr(kv), _ptr(idx_out),
                                     _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse, idx_out


def dsa_timing_begin() -> None:
    """Start a kernel-timing session: the library brackets each of its kernel
    launches with HIP events on the launch's stream."""
    _check(lib().dsa_timing_begin())


def dsa_timing_end(max_kernels: int = 32) -> dict:
    """End the session; {kernel name: {launches, dropped, total_ms, min_ms,
    max_ms, avg_us}} in order of first launch."""
    recs = (DsaKernelTime * max_kernels)()
    n = ctypes.c_int32(0)
    _check(lib().dsa_timing_end(recs, max_kernels, ctypes.byref(n)))
    out = {}
    for r in recs[:min(n.value, max_kernels)]:
        out[r.name.decode()] = dict(launches=r.launches, dropped=r.dropped, total_ms=r.total_ms,
                                    min_ms=r.min_ms, max_ms=r.max_ms,
                                    avg_us=1e3 * r.total_ms / r.launches if r.launches else None)
    return out


_DT_OF = {torch.bfloat16: DSA_BF16, torch.float32: DSA_F32, torch.uint8: DSA_FP8_E4M3}


def dsa_cache_fill(x, W, kv_gamma, k_gamma, k_beta, rope_cos, rope_sin, slots, kv_cache, k_cache,
                   k_sf=None, w_out: Optional[torch.Tensor] = None,
                   w_dtype=torch.bfloat16, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Cache fill and indexer inputs of N tokens: writes rows slots[n] of
    kv_cache [rows, 576] (bf16 / fp32) and k_cache [rows, 128] (bf16 / fp32,
    or uint8 E4M3 codes with k_sf [rows] ue8m0 scales); returns the head
    weights w [N, 64]."""
    N, D = x.shape
    dev = x.device
    _req(x, "x", (N, D), (torch.bfloat16,), dev)
    _req(W, "W", (768, D), (torch.bfloat16,), dev)
    _req(kv_gamma, "kv_gamma", (512,), (torch.float32,), dev)
    _req(k_gamma, "k_gamma", (128,), (torch.float32,), dev)
    _req(k_beta, "k_beta", (128,), (torch.float32,), dev)
    _req(rope_cos, "rope_cos", (N, 32), (torch.float32,), dev)
    _req(rope_sin, "rope_sin", (N, 32), (torch.float32,), dev)
    _req(slots, "slots", (N,), (torch.int64,), dev)
    _req(kv_cache, "kv_cache", (kv_cache.shape[0], 576), (torch.bfloat16, torch.float32), dev)
    _req(k_cache, "k_cache", (k_cache.shape[0], 128), (torch.bfloat16, torch.float32, torch.uint8),
         dev)
    if k_cache.dtype == torch.uint8:
        _req(k_sf, "k_sf", (k_cache.shape[0],), (torch.uint8,), dev)
    if w_out is None:
        w_out = torch.empty((N, 64), dtype=w_dtype, device=dev)
    _req(w_out, "w_out", (N, 64), (torch.bfloat16, torch.float32), dev)
    if ws is None:
        nb = lib().dsa_cache_fill_workspace_bytes(N, D)
        if nb == ctypes.c_size_t(-1).value:
            raise DsaError(1, f"cache fill: invalid sizes N={N}, D={D}")
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib().dsa_cache_fill(N, D, _ptr(x), _ptr(W), _ptr(kv_gamma), _ptr(k_gamma),
                                _ptr(k_beta), _ptr(rope_cos), _ptr(rope_sin), _ptr(slots),
                                _DT_OF[kv_cache.dtype], _ptr(kv_cache), _DT_OF[k_cache.dtype],
                                _ptr(k_cache), _ptr(k_sf), _DT_OF[w_out.dtype], _ptr(w_out),
                                _ptr(ws), _ws_bytes(ws, dev), _stream(dev)))
    return w_out


def dsa_indexer_query(cq, wq_b, q_dtype=torch.bfloat16, q_out: Optional[torch.Tensor] = None,
                      q_sf: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Indexer query Q^I = c^Q wq_b of N tokens: q [N, 64, 128] (bf16 / fp32, or
    uint8 E4M3 codes) and, for E4M3, q_sf [N, 64] ue8m0 scales (else None)."""
    N, Dq = cq.shape
    dev = cq.device
    _req(cq, "cq", (N, Dq), (torch.bfloat16,), dev)
    _req(wq_b, "wq_b", (8192, Dq), (torch.bfloat16,), dev)
    fp8 = q_dtype == torch.uint8
    if q_out is None:
        q_out = torch.empty((N, 64, 128), dtype=q_dtype, device=dev)
    _req(q_out, "q_out", (N, 64, 128), (torch.bfloat16, torch.float32, torch.uint8), dev)
    if fp8 and q_sf is None:
        q_sf = torch.empty((N, 64), dtype=torch.uint8, device=dev)
    if q_sf is not None:
        _req(q_sf, "q_sf", (N, 64), (torch.uint8,), dev)
    if ws is None:
        nb = lib().dsa_indexer_query_workspace_bytes(N, Dq)
        if nb == ctypes.c_size_t(-1).value:
            raise DsaError(1, f"indexer query: invalid sizes N={N}, Dq={Dq}")
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib().dsa_indexer_query(N, Dq, _ptr(cq), _ptr(wq_b), _DT_OF[q_out.dtype], _ptr(q_out),
                                   _ptr(q_sf), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)))
    return q_out, (q_sf if fp8 else None)


def dsa_absorb_prepare(kv_b, w_uk_t: Optional[torch.Tensor] = None):
    """W_UK of kv_b_proj's weight kv_b [H * 256, 512] in the form
    dsa_absorb_query reads: w_uk_t [H, 512, 128], w_uk_t[h, c, e] = kv_b[256 h + e, c]."""
    R, C = kv_b.shape
    if R % 256 or C != 512:
        raise ValueError(f"kv_b has shape {tuple(kv_b.shape)}, expected [H * 256, 512]")
    H = R // 256
    dev = kv_b.device
    _req(kv_b, "kv_b", (R, 512), (torch.bfloat16,), dev)
    if w_uk_t is None:
        w_uk_t = torch.empty((H, 512, 128), dtype=torch.bfloat16, device=dev)
    _req(w_uk_t, "w_uk_t", (H, 512, 128), (torch.bfloat16,), dev)
    _check(lib().dsa_absorb_prepare(H, _ptr(kv_b), _ptr(w_uk_t), _stream(dev)))
    return w_uk_t


def dsa_absorb_query(qb, w_uk_t, rope_cos, rope_sin, q_dtype=torch.bfloat16,
                     q: Optional[torch.Tensor] = None):
    """The sparse attention's query [N, H, 576] from q_b_proj's output qb
    [N, H, 192]: the latent part q^C_h absorbed through W_UK,h, the rotary part
    turned by the tokens' angles (rope_cos, rope_sin [N, 32])."""
    N, H, _ = qb.shape
    dev = qb.device
    _req(qb, "qb", (N, H, 192), (torch.bfloat16,), dev)
    _req(w_uk_t, "w_uk_t", (H, 512, 128), (torch.bfloat16,), dev)
    _req(rope_cos, "rope_cos", (N, 32), (torch.float32,), dev)
    _req(rope_sin, "rope_sin", (N, 32), (torch.float32,), dev)
    if q is None:
        q = torch.empty((N, H, 576), dtype=q_dtype, device=dev)
    _req(q, "q", (N, H, 576), (torch.bfloat16, torch.float32), dev)
    _check(lib().dsa_absorb_query(N, H, _ptr(qb), _ptr(w_uk_t), _ptr(rope_cos), _ptr(rope_sin),
                                  _DT_OF[q.dtype], _ptr(q), _stream(dev)))
    return q


def dsa_absorb_output(o_lat, kv_b, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Head outputs [N, H * 128] from the latent contexts o_lat [N, H, 512]
    through each head's W_UV (the value half of kv_b [H * 256, 512])."""
    N, H, _ = o_lat.shape
    dev = o_lat.device
    _req(o_lat, "o_lat", (N, H, 512), (torch.bfloat16,), dev)
    _req(kv_b, "kv_b", (H * 256, 512), (torch.bfloat16,), dev)
    if out is None:
        out = torch.empty((N, H * 128), dtype=out_dtype, device=dev)
    _req(out, "out", (N, H * 128), (torch.bfloat16, torch.float32), dev)
    _check(lib().dsa_absorb_output(N, H, _ptr(o_lat), _ptr(kv_b), _DT_OF[out.dtype], _ptr(out),
                                   _stream(dev)))
    return out


def dsa_output_projection(premix, wo, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """out [N, Dout] = premix [N, Din] wo^T (wo [Dout, Din] in Linear layout)."""
    N, Din = premix.shape
    Dout = wo.shape[0]
    dev = premix.device
    _req(premix, "premix", (N, Din), (torch.bfloat16,), dev)
    _req(wo, "wo", (Dout, Din), (torch.bfloat16,), dev)
    if out is None:
        out = torch.empty((N, Dout), dtype=out_dtype, device=dev)
    _req(out, "out", (N, Dout), (torch.bfloat16, torch.float32), dev)
    if ws is None:
        nb = lib().dsa_output_projection_workspace_bytes(N, Din, Dout)
        if nb == ctypes.c_size_t(-1).value:
            raise DsaError(1, f"output projection: invalid sizes N={N}, Din={Din}, Dout={Dout}")
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib().dsa_output_projection(N, Din, Dout, _ptr(premix), _ptr(wo), _DT_OF[out.dtype],
                                       _ptr(out), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)))
    return out

"""CPU oracle for the sparse-attention hot path (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it and shares no code with it.

The arithmetic lives in ``dsa_oracle.c`` (plain fp64 loops; see its header for
the passages each routine follows and the readings taken where the pages are
silent).  This module only marshals numpy arrays and spreads query rows over
host threads; ctypes releases the GIL while the C routine runs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = [os.path.join(_HERE, "dsa_oracle.c")]

DT_CODE = {"f32": 0, "bf16": 1, "fp8": 2}


def build(force: bool = True, cc: str = "gcc", extra: Sequence[str] = (),
          src: Optional[str] = None, out: Optional[str] = None) -> str:
    """Compile the oracle into a shared library (plain C, -O2)."""
    src = src or _SOURCES[0]
    out = out or LIB_PATH
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-I", _HERE, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "S", "HI", "DI", "H", "Dc", "Dr", "K")] + [
        ("idx_scale", ctypes.c_float), ("sm_scale", ctypes.c_float),
        ("idx_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("mla_dtype", ctypes.c_int32)]


_lib_lock = threading.Lock()
_libs = {}


def load(path: Optional[str] = None):
    path = path or LIB_PATH
    with _lib_lock:
        if path not in _libs:
            if path == LIB_PATH and not os.path.exists(path):
                build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i32 = ctypes.c_int32
            sp = ctypes.POINTER(_Shape)
            lib.orc_indexer_scores.argtypes = [sp, i32, P, P, P, P, P, P, P, P]
            lib.orc_indexer_scores_ragged.argtypes = [sp, i32, P, P, P, P, P, P, P, P, P]
            lib.orc_topk.argtypes = [sp, i32, P, P]
            lib.orc_sparse_mla.argtypes = [sp, i32, P, P, P, P, i32, P, P, P]
            lib.orc_dense_mla.argtypes = [sp, i32, P, P, P, P, P, P]
            lib.orc_explicit_mla.argtypes = [i32] * 6 + [ctypes.c_double] + [P] * 7
            lib.orc_cache_fill.argtypes = [i32, i32] + [P] * 10
            lib.orc_quantize_e4m3_block.argtypes = [P, i32, P, P]
            lib.orc_indexer_query.argtypes = [i32, i32, P, P, i32, P]
            lib.orc_absorb_query.argtypes = [i32] * 6 + [P] * 5
            lib.orc_absorb_output.argtypes = [i32] * 5 + [P] * 3
            lib.orc_linear_bf16.argtypes = [i32, i32, i32, P, P, P]
            for f in ("orc_indexer_scores", "orc_indexer_scores_ragged", "orc_topk", "orc_sparse_mla", "orc_dense_mla",
                      "orc_explicit_mla", "orc_cache_fill", "orc_quantize_e4m3_block",
                      "orc_indexer_query", "orc_absorb_query", "orc_absorb_output",
                      "orc_linear_bf16"):
                getattr(lib, f).restype = ctypes.c_int
            _libs[path] = lib
        return _libs[path]


def shape_of(cfg) -> _Shape:
    return _Shape(cfg.B, cfg.T, cfg.S, cfg.HI, cfg.DI, cfg.H, cfg.Dc, cfg.Dr, cfg.K,
                  cfg.index_scale, cfg.softmax_scale, DT_CODE[cfg.idx_dtype],
                  DT_CODE[cfg.w_dtype], DT_CODE[cfg.mla_dtype])


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _split(n: int, threads: int):
    threads = max(1, min(threads, n))
    step = (n + threads - 1) // threads
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def _run_rows(fn, n, threads):
    chunks = _split(n, threads) if n > 0 else []
    if len(chunks) <= 1:
        for lo, hi in chunks:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        list(ex.map(lambda c: fn(*c), chunks))


def indexer_scores(cfg, row_b, row_t, q_idx_rows, w_rows, k_idx, q_sf_rows=None, k_sf=None,
                   threads: Optional[int] = None, lib=None, seq_lens=None) -> np.ndarray:
    """Index scores of the given query rows, [n, S] fp32 (future keys -inf).
    seq_lens [B] (optional): per-sequence context lengths (ragged batch)."""
    lib = lib or load()
    sh = shape_of(cfg)
    row_b = _c(row_b, np.int32)
    row_t = _c(row_t, np.int32)
    n = row_b.shape[0]
    q_idx_rows, w_rows, k_idx = _c(q_idx_rows), _c(w_rows), _c(k_idx)
    q_sf_rows, k_sf = _c(q_sf_rows, np.uint8), _c(k_sf, np.uint8)
    out = np.empty((n, cfg.S), np.float32)
    qrow = cfg.HI * cfg.DI
    nblk = cfg.DI // 128 if cfg.idx_dtype == "fp8" else 0
    lens = _c(seq_lens, np.int32)

    def run(lo, hi):
        rc = lib.orc_indexer_scores_ragged(
            ctypes.byref(sh), hi - lo, row_b[lo:].ctypes.data, row_t[lo:].ctypes.data, _ptr(lens),
            q_idx_rows.ctypes.data + lo * qrow * q_idx_rows.itemsize,
            None if q_sf_rows is None else q_sf_rows.ctypes.data + lo * cfg.HI * nblk,
            _ptr(k_idx), _ptr(k_sf),
            w_rows.ctypes.data + lo * cfg.HI * w_rows.itemsize,
            out[lo:].ctypes.data)
        if rc:
            raise ValueError("orc_indexer_scores rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return out


def topk(cfg, scores, threads: Optional[int] = None, lib=None) -> np.ndarray:
    """Top-K index rows [n, min(K, S)] int32 (ascending, -1 padded)."""
    lib = lib or load()
    sh = shape_of(cfg)
    scores = _c(scores, np.float32)
    n = scores.shape[0]
    assert scores.shape[1] == cfg.S
    out = np.empty((n, cfg.K_eff), np.int32)

    def run(lo, hi):
        if lib.orc_topk(ctypes.byref(sh), hi - lo, scores[lo:].ctypes.data, out[lo:].ctypes.data):
            raise ValueError("orc_topk rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return out


def sparse_mla(cfg, row_b, q_rows, kv, idx, want_probs: bool = False,
               threads: Optional[int] = None, lib=None):
    """Absorbed sparse latent attention: (o [n,H,Dc] f64, lse [n,H] f64[, probs])."""
    lib = lib or load()
    sh = shape_of(cfg)
    row_b = _c(row_b, np.int32)
    q_rows, kv, idx = _c(q_rows), _c(kv), _c(idx, np.int32)
    n, W = idx.shape
    o = np.empty((n, cfg.H, cfg.Dc), np.float64)
    lse = np.empty((n, cfg.H), np.float64)
    probs = np.empty((n, cfg.H, W), np.float64) if want_probs else None
    qrow = cfg.H * cfg.D * q_rows.itemsize

    def run(lo, hi):
        rc = lib.orc_sparse_mla(
            ctypes.byref(sh), hi - lo, row_b[lo:].ctypes.data, q_rows.ctypes.data + lo * qrow,
            kv.ctypes.data, idx[lo:].ctypes.data, W, o[lo:].ctypes.data, lse[lo:].ctypes.data,
            None if probs is None else probs[lo:].ctypes.data)
        if rc:
            raise ValueError("orc_sparse_mla rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return (o, lse, probs) if want_probs else (o, lse)


def dense_mla(cfg, row_b, row_t, q_rows, kv, threads: Optional[int] = None, lib=None):
    """Dense causal latent attention: (o [n,H,Dc] f64, lse [n,H] f64)."""
    lib = lib or load()
    sh = shape_of(cfg)
    row_b, row_t = _c(row_b, np.int32), _c(row_t, np.int32)
    q_rows, kv = _c(q_rows), _c(kv)
    n = row_b.shape[0]
    o = np.empty((n, cfg.H, cfg.Dc), np.float64)
    lse = np.empty((n, cfg.H), np.float64)
    qrow = cfg.H * cfg.D * q_rows.itemsize

    def run(lo, hi):
        rc = lib.orc_dense_mla(ctypes.byref(sh), hi - lo, row_b[lo:].ctypes.data,
                               row_t[lo:].ctypes.data, q_rows.ctypes.data + lo * qrow,
                               kv.ctypes.data, o[lo:].ctypes.data, lse[lo:].ctypes.data)
        if rc:
            raise ValueError("orc_dense_mla rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return o, lse


def explicit_mla(qC, qR, c, r, W_UK, W_UV, sm_scale, lib=None) -> np.ndarray:
    """Explicit (non-absorbed) latent attention of one query, fp64: out [H, Dv]."""
    lib = lib or load()
    qC, qR, c, r = (_c(a, np.float64) for a in (qC, qR, c, r))
    W_UK, W_UV = _c(W_UK, np.float64), _c(W_UV, np.float64)
    H, Dn = qC.shape
    Dr = qR.shape[1]
    nkeys, Dc = c.shape
    Dv = W_UV.shape[1] // H
    out = np.empty((H, Dv), np.float64)
    rc = lib.orc_explicit_mla(H, Dc, Dn, Dv, Dr, nkeys, float(sm_scale), qC.ctypes.data,
                              qR.ctypes.data, c.ctypes.data, r.ctypes.data, W_UK.ctypes.data,
                              W_UV.ctypes.data, out.ctypes.data)
    if rc:
        raise ValueError("orc_explicit_mla rejected its arguments")
    return out


FILL_COLS = 768  # 512 latent + 64 rotary + 128 indexer key + 64 head weights


def cache_fill(x_bits, W_bits, kv_gamma, k_gamma, k_beta, rope_cos, rope_sin,
               threads: Optional[int] = None, lib=None):
    """Cache fill and indexer inputs of n tokens: (kv [n, 576], k^I [n, 128],
    w [n, 64]) in fp64, before any rounding to a storage format.  x_bits
    [n, D] and W_bits [768, D] are bf16 bit patterns (uint16)."""
    lib = lib or load()
    x_bits = _c(x_bits, np.uint16)
    W_bits = _c(W_bits, np.uint16)
    n, D = x_bits.shape
    assert W_bits.shape == (FILL_COLS, D)
    kv_gamma, k_gamma, k_beta = (_c(a, np.float32) for a in (kv_gamma, k_gamma, k_beta))
    rope_cos, rope_sin = _c(rope_cos, np.float32), _c(rope_sin, np.float32)
    assert rope_cos.shape == (n, 32) and rope_sin.shape == (n, 32)
    kv = np.empty((n, 576), np.float64)
    k = np.empty((n, 128), np.float64)
    w = np.empty((n, 64), np.float64)

    def run(lo, hi):
        rc = lib.orc_cache_fill(hi - lo, D, x_bits[lo:].ctypes.data, W_bits.ctypes.data,
                                kv_gamma.ctypes.data, k_gamma.ctypes.data, k_beta.ctypes.data,
                                rope_cos[lo:].ctypes.data, rope_sin[lo:].ctypes.data,
                                kv[lo:].ctypes.data, k[lo:].ctypes.data, w[lo:].ctypes.data)
        if rc:
            raise ValueError("orc_cache_fill rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return kv, k, w


def quantize_e4m3(y, block: int = 128, lib=None):
    """ue8m0 + E4M3 block quantisation of fp64 values [..., m * block]:
    (codes uint8 [..., m * block], scale bytes uint8 [..., m])."""
    lib = lib or load()
    y = _c(y, np.float64)
    flat = y.reshape(-1, block)
    codes = np.empty(flat.shape, np.uint8)
    sb = np.empty(flat.shape[0], np.uint8)
    for i in range(flat.shape[0]):
        if lib.orc_quantize_e4m3_block(flat[i].ctypes.data, block, codes[i].ctypes.data,
                                       sb[i:].ctypes.data):
            raise ValueError("orc_quantize_e4m3_block rejected its arguments")
    return codes.reshape(y.shape), sb.reshape(y.shape[:-1] + (y.shape[-1] // block,))


def indexer_query(cq_bits, wqb_bits, threads: Optional[int] = None, lib=None):
    """Indexer query Q^I = c^Q wq_b of n tokens: [n, out_dim] fp64 (cq_bits
    [n, Dq], wqb_bits [out_dim, Dq] bf16 bit patterns)."""
    lib = lib or load()
    cq_bits = _c(cq_bits, np.uint16)
    wqb_bits = _c(wqb_bits, np.uint16)
    n, Dq = cq_bits.shape
    out_dim = wqb_bits.shape[0]
    q = np.empty((n, out_dim), np.float64)

    def run(lo, hi):
        if lib.orc_indexer_query(hi - lo, Dq, cq_bits[lo:].ctypes.data, wqb_bits.ctypes.data,
                                 out_dim, q[lo:].ctypes.data):
            raise ValueError("orc_indexer_query rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return q


def absorb_query(qb, kv_b, rope_cos, rope_sin, Dn: int = 128, threads: Optional[int] = None,
                 lib=None) -> np.ndarray:
    """The sparse attention's query from q_b_proj's output, fp64: qb [n, H,
    Dn + Dr], kv_b [H (Dn + Dv), Dc], rope_cos / rope_sin [n, Dr / 2] ->
    q [n, H, Dc + Dr] (latent part absorbed through W_UK, rotary part turned)."""
    lib = lib or load()
    qb = _c(qb, np.float64)
    kv_b = _c(kv_b, np.float64)
    rope_cos, rope_sin = _c(rope_cos, np.float64), _c(rope_sin, np.float64)
    n, H, in_w = qb.shape
    Dr = in_w - Dn
    Dc = kv_b.shape[1]
    Dv = kv_b.shape[0] // H - Dn
    assert kv_b.shape[0] == H * (Dn + Dv) and rope_cos.shape == (n, Dr // 2)
    q = np.empty((n, H, Dc + Dr), np.float64)

    def run(lo, hi):
        if lib.orc_absorb_query(hi - lo, H, Dc, Dn, Dv, Dr, qb[lo:].ctypes.data, kv_b.ctypes.data,
                                rope_cos[lo:].ctypes.data, rope_sin[lo:].ctypes.data,
                                q[lo:].ctypes.data):
            raise ValueError("orc_absorb_query rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return q


def absorb_output(o, kv_b, Dn: int = 128, threads: Optional[int] = None, lib=None) -> np.ndarray:
    """Head outputs from latent contexts, fp64: o [n, H, Dc], kv_b [H (Dn +
    Dv), Dc] -> out [n, H Dv] (each head through its W_UV half)."""
    lib = lib or load()
    o = _c(o, np.float64)
    kv_b = _c(kv_b, np.float64)
    n, H, Dc = o.shape
    Dv = kv_b.shape[0] // H - Dn
    assert kv_b.shape == (H * (Dn + Dv), Dc)
    out = np.empty((n, H * Dv), np.float64)

    def run(lo, hi):
        if lib.orc_absorb_output(hi - lo, H, Dc, Dn, Dv, o[lo:].ctypes.data, kv_b.ctypes.data,
                                 out[lo:].ctypes.data):
            raise ValueError("orc_absorb_output rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return out


def linear_bf16(x_bits, W_bits, threads: Optional[int] = None, lib=None) -> np.ndarray:
    """A Linear layer (o_proj / wo) on bf16 bit patterns: x [n, Din], W [Dout,
    Din] -> x W^T [n, Dout] in fp64."""
    lib = lib or load()
    x_bits = _c(x_bits, np.uint16)
    W_bits = _c(W_bits, np.uint16)
    n, Din = x_bits.shape
    Dout = W_bits.shape[0]
    assert W_bits.shape == (Dout, Din)
    out = np.empty((n, Dout), np.float64)

    def run(lo, hi):
        if lib.orc_linear_bf16(hi - lo, Din, Dout, x_bits[lo:].ctypes.data, W_bits.ctypes.data,
                               out[lo:].ctypes.data):
            raise ValueError("orc_linear_bf16 rejected its arguments")

    _run_rows(run, n, threads or default_threads())
    return out

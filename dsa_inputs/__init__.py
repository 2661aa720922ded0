"""Seeded synthetic inputs for the sparse-attention hot path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no part of the method's arithmetic (no scores, no
selection, no attention): it only draws numbers, rounds them to the storage
formats, and shapes them the way the workloads are described.

Workloads (shapes from the DeepSeek-V3.2 pages: 64 indexer heads of width 128,
top-2048, 128 MLA heads over a 512-wide latent plus a 64-wide rotary key):

* ``tiny``          fp32 causal prefill, T = S = 256, integer inputs in [-3, 3].
* ``decode_8k``     bf16 decode, batch 32, one query per sequence, 8192 keys.
* ``prefill_16k``   bf16 causal prefill, batch 1, T = S = 16384.
* ``decode_128k``   bf16 decode, batch 8, 131072 keys, a planted key cluster.
* ``decode_64k_fp8`` e4m3 indexer (ue8m0 block scales), batch 64, 65536 keys.

Every tensor is drawn in blocks of ``ROW_BLOCK`` rows, each block from its own
``numpy.random.default_rng([seed, tensor_id, batch, block])`` stream.  A block
can therefore be regenerated on its own, which lets the oracle rebuild the rows
it samples from a large workload without materialising the whole tensor.

Storage formats:
* bf16 is kept as ``uint16`` bit patterns (round-to-nearest-even from fp32);
* fp8 is OCP E4M3FN bytes (``uint8``) with one ue8m0 scale byte per 128-element
  block (value = e4m3 * 2**(byte - 127));
* fp32 is ``float32``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

ROW_BLOCK = 256

F32, BF16, FP8 = "f32", "bf16", "fp8"

# tensor ids for the counter-based streams
_TID = {"q_idx": 0, "k_idx": 1, "w": 2, "q": 3, "kv": 4, "cluster": 5}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    S: int
    HI: int
    DI: int
    H: int
    Dc: int
    Dr: int
    K: int
    idx_dtype: str
    w_dtype: str
    mla_dtype: str
    seed: int
    integer: bool = False
    cluster: int = 0          # planted cluster size per sequence (0 = none)
    idx_scale: Optional[float] = None
    sm_scale: Optional[float] = None

    @property
    def K_eff(self) -> int:
        return min(self.K, self.S)

    @property
    def D(self) -> int:
        return self.Dc + self.Dr

    @property
    def index_scale(self) -> float:
        # 1/(sqrt(HI) * sqrt(DI)): the prefactor of the index score
        if self.idx_scale is not None:
            return self.idx_scale
        return float(np.float32(1.0 / (math.sqrt(self.HI) * math.sqrt(self.DI))))

    @property
    def softmax_scale(self) -> float:
        if self.sm_scale is not None:
            return self.sm_scale
        return float(np.float32(1.0 / math.sqrt(self._qk_head_dim())))

    def _qk_head_dim(self) -> int:
        # V3.2 shapes: qk_head_dim = 128 (nope) + 64 (rope) = 192.  The tiny
        # workload states no scale; its reading is 1/sqrt(Dc + Dr).
        if (self.H, self.Dc, self.Dr) == (128, 512, 64):
            return 192
        return self.Dc + self.Dr

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def q_pos(self, t: int) -> int:
        return self.S - self.T + t


_V32 = dict(HI=64, DI=128, H=128, Dc=512, Dr=64, K=2048)

CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", B=1, T=256, S=256, HI=4, DI=32, H=4, Dc=64, Dr=16, K=32,
                   idx_dtype=F32, w_dtype=F32, mla_dtype=F32, seed=0, integer=True),
    "decode_8k": Config("decode_8k", B=32, T=1, S=8192, idx_dtype=BF16, w_dtype=BF16,
                        mla_dtype=BF16, seed=1, **_V32),
    "prefill_16k": Config("prefill_16k", B=1, T=16384, S=16384, idx_dtype=BF16,
                          w_dtype=BF16, mla_dtype=BF16, seed=2, **_V32),
    "decode_128k": Config("decode_128k", B=8, T=1, S=131072, idx_dtype=BF16,
                          w_dtype=BF16, mla_dtype=BF16, seed=3, cluster=4096, **_V32),
    "decode_64k_fp8": Config("decode_64k_fp8", B=64, T=1, S=65536, idx_dtype=FP8,
                             w_dtype=BF16, mla_dtype=BF16, seed=4, **_V32),
    # the prefill with the checkpoint's indexer format (e4m3 codes, ue8m0
    # block scales): prefill_16k's shapes and draws, quantised like decode_64k_fp8
    "prefill_16k_fp8": Config("prefill_16k_fp8", B=1, T=16384, S=16384, idx_dtype=FP8,
                              w_dtype=BF16, mla_dtype=BF16, seed=5, **_V32),
}


# ----------------------------------------------------------------------------
# storage-format conversions (no method arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x8000 cannot wrap for any non-NaN pattern (the largest, -inf, is
    # 0xff800000); NaN lanes are overwritten below
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_to_f32(c: np.ndarray) -> np.ndarray:
    """OCP E4M3FN byte -> fp32 (exact)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int32)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 0xF) & (m == 0x7), np.nan, v)
    return (s * v).astype(np.float32)


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN byte, round to nearest even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float32)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x).astype(np.float32)
    a = np.minimum(a, np.float32(448.0))
    bits = a.view(np.uint32).astype(np.uint64)
    # normal range (|a| >= 2^-6): keep 3 mantissa bits, round half to even
    lsb = (bits >> 20) & 1
    rb = bits + 0x7FFFF + lsb
    e8 = (rb >> 23).astype(np.int64) - 127 + 7
    m8 = ((rb >> 20) & 7).astype(np.int64)
    over = (e8 > 15) | ((e8 == 15) & (m8 == 7))
    e8 = np.where(over, 15, e8)
    m8 = np.where(over, 6, m8)
    normal_code = (e8 << 3) | m8
    # subnormal range (|a| < 2^-6): step 2^-9, np.rint rounds half to even
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)  # 0..8
    code = np.where(a < np.float32(2.0 ** -6), sub, normal_code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_e4m3_blocks(x: np.ndarray, block: int = 128):
    """Per-``block`` ue8m0 scale (2**ceil(log2(amax/448))) and e4m3 bytes.

    Returns (codes uint8 [..., n], scale bytes uint8 [..., n // block]).
    An all-zero block gets scale byte 127 (scale 1).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % block == 0
    xb = x.reshape(x.shape[:-1] + (n // block, block))
    amax = np.abs(xb).max(axis=-1).astype(np.float64)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.ceil(np.log2(amax / 448.0)), 0.0)
    ex = np.clip(ex, -127, 127).astype(np.int64)
    sbyte = (ex + 127).astype(np.uint8)
    scale = np.exp2(ex.astype(np.float64))
    codes = f32_to_e4m3((xb / scale[..., None]).astype(np.float32))
    return codes.reshape(x.shape), sbyte


def ue8m0_to_f32(b: np.ndarray) -> np.ndarray:
    return np.exp2(np.asarray(b, dtype=np.float64) - 127.0).astype(np.float32)


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------

def _rng(cfg: Config, tensor: str, b: int, blk: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, _TID[tensor], b, blk])


def _shape_tail(cfg: Config, tensor: str):
    return {"q_idx": (cfg.HI, cfg.DI), "k_idx": (cfg.DI,), "w": (cfg.HI,),
            "q": (cfg.H, cfg.D), "kv": (cfg.D,)}[tensor]


def _nrows(cfg: Config, tensor: str) -> int:
    return cfg.T if tensor in ("q_idx", "w", "q") else cfg.S


def _draw_block_f32(cfg: Config, tensor: str, b: int, blk: int) -> np.ndarray:
    """fp32 values of rows [blk*ROW_BLOCK, ...) of ``tensor`` for sequence b."""
    n = _nrows(cfg, tensor)
    r0 = blk * ROW_BLOCK
    r1 = min(n, r0 + ROW_BLOCK)
    shape = (r1 - r0,) + _shape_tail(cfg, tensor)
    g = _rng(cfg, tensor, b, blk)
    if cfg.integer:
        return g.integers(-3, 4, size=shape).astype(np.float32)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if tensor == "w":
        x = x / np.float32(8.0)
    elif tensor == "kv":
        # latent part is RMS-normalised (unit gain, eps 1e-6, fp32), the rotary
        # key is left as drawn
        lat = x[:, : cfg.Dc]
        ms = np.mean(lat.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32)
        x[:, : cfg.Dc] = lat / np.sqrt(ms + np.float32(1e-6), dtype=np.float32)
    return x


def _store(x: np.ndarray, dtype: str):
    if dtype == F32:
        return x.astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _cluster_direction(cfg: Config, b: int) -> np.ndarray:
    """Unit vector along sum_h w_h * Q^I_h of the sequence's last query."""
    t = cfg.T - 1
    qb = rows(cfg, "q_idx", b, t, t + 1)
    wb = rows(cfg, "w", b, t, t + 1)
    qv = decode_values(cfg, "q_idx", qb)[0].astype(np.float64)
    wv = decode_values(cfg, "w", wb)[0].astype(np.float64)
    u = (wv[:, None] * qv).sum(axis=0)
    return u / np.linalg.norm(u)


def cluster_positions(cfg: Config, b: int) -> np.ndarray:
    if cfg.cluster <= 0:
        return np.zeros(0, dtype=np.int64)
    g = _rng(cfg, "cluster", b, 0)
    return np.sort(g.choice(cfg.S, size=cfg.cluster, replace=False))


def rows(cfg: Config, tensor: str, b: int, r0: int, r1: int):
    """Rows [r0, r1) of ``tensor`` for sequence ``b`` in storage format.

    For fp8 indexer tensors the result is a tuple (codes, scale_bytes).
    """
    n = _nrows(cfg, tensor)
    assert 0 <= r0 <= r1 <= n
    parts = []
    blocks = range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1) if r1 > r0 else range(0)
    for blk in blocks:
        x = _draw_block_f32(cfg, tensor, b, blk)
        base = blk * ROW_BLOCK
        lo, hi = max(r0, base) - base, min(r1, base + x.shape[0]) - base
        x = x[lo:hi]
        if tensor == "k_idx" and cfg.cluster > 0:
            pos = cluster_positions(cfg, b)
            sel = pos[(pos >= base + lo) & (pos < base + hi)] - (base + lo)
            if sel.size:
                u = _cluster_direction(cfg, b).astype(np.float32)
                x = x.copy()
                x[sel] += np.float32(3.0) * u
        parts.append(x)
    x = np.concatenate(parts, axis=0) if parts else np.zeros(
        (0,) + _shape_tail(cfg, tensor), np.float32)
    if tensor in ("q_idx", "k_idx"):
        if cfg.idx_dtype == FP8:
            if cfg.integer:
                # integers in [-3, 3] are exact in e4m3; scale byte 127 (x1)
                codes = f32_to_e4m3(x)
                sb = np.full(x.shape[:-1] + (cfg.DI // 128,), 127, np.uint8)
                return codes, sb
            return quantize_e4m3_blocks(x, 128)
        return _store(x, cfg.idx_dtype)
    if tensor == "w":
        return _store(x, cfg.w_dtype)
    return _store(x, cfg.mla_dtype)


def decode_values(cfg: Config, tensor: str, stored) -> np.ndarray:
    """Storage format -> fp32 values (exact)."""
    if tensor in ("q_idx", "k_idx") and cfg.idx_dtype == FP8:
        codes, sb = stored
        v = e4m3_to_f32(codes)
        sc = ue8m0_to_f32(sb)
        vb = v.reshape(v.shape[:-1] + (sc.shape[-1], -1))
        return (vb * sc[..., None]).reshape(v.shape)
    dt = {"q_idx": cfg.idx_dtype, "k_idx": cfg.idx_dtype, "w": cfg.w_dtype,
          "q": cfg.mla_dtype, "kv": cfg.mla_dtype}[tensor]
    if dt == BF16:
        return bf16_bits_to_f32(stored)
    return np.asarray(stored, dtype=np.float32)


def full(cfg: Config, tensor: str):
    """The whole ``tensor`` as [B, n, ...] in storage format (host memory)."""
    n = _nrows(cfg, tensor)
    per_b = [rows(cfg, tensor, b, 0, n) for b in range(cfg.B)]
    if isinstance(per_b[0], tuple):
        return (np.stack([p[0] for p in per_b]), np.stack([p[1] for p in per_b]))
    return np.stack(per_b)


def iter_blocks(cfg: Config, tensor: str, values_per_chunk: int = 1 << 24, threads: int = 0):
    """Yield (b, r0, r1, stored) chunks covering ``tensor`` in order, each
    about ``values_per_chunk`` values (bounded memory).  Chunks are drawn by
    ``threads`` worker threads (0 = up to 16); the draws do not depend on it."""
    import concurrent.futures as cf
    import os
    n = _nrows(cfg, tensor)
    row_vals = int(np.prod(_shape_tail(cfg, tensor)))
    step = max(ROW_BLOCK, (values_per_chunk // row_vals // ROW_BLOCK) * ROW_BLOCK)
    jobs = [(b, r0, min(n, r0 + step)) for b in range(cfg.B) for r0 in range(0, n, step)]
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or len(jobs) <= 1:
        for b, r0, r1 in jobs:
            yield b, r0, r1, rows(cfg, tensor, b, r0, r1)
        return
    with cf.ThreadPoolExecutor(threads) as ex:
        pending = []
        it = iter(jobs)
        for job in it:
            pending.append((job, ex.submit(rows, cfg, tensor, *job)))
            if len(pending) >= 2 * threads:
                break
        while pending:
            (b, r0, r1), fut = pending.pop(0)
            nxt = next(it, None)
            if nxt is not None:
                pending.append((nxt, ex.submit(rows, cfg, tensor, *nxt)))
            yield b, r0, r1, fut.result()

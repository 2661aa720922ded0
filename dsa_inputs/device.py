"""Device-side plumbing for the seeded inputs: upload a workload's tensors to
the GPU, read results back, and build the C ABI's shape struct from a
workload.  Like the rest of ``dsa_inputs`` it holds none of the method's
arithmetic; the tests and the benchmark both use it."""
from __future__ import annotations

import numpy as np

from . import iter_blocks

_DT = {"f32": 0, "bf16": 1, "fp8": 2}


def torch():
    import torch as _t
    return _t


def shape_of(cfg):
    """The dsa_shape_t of a workload (through the package's binding)."""
    import sparse_latent_attention_lightning_amd as dsa
    return dsa.make_shape(cfg.B, cfg.T, cfg.S, cfg.HI, cfg.DI, cfg.H, cfg.Dc, cfg.Dr, cfg.K,
                          cfg.index_scale, cfg.softmax_scale, _DT[cfg.idx_dtype],
                          _DT[cfg.w_dtype], _DT[cfg.mla_dtype])


def to_dev(arr, dtype_name, device="cuda"):
    t = torch()
    arr = np.ascontiguousarray(arr)
    if dtype_name == "bf16":
        return t.from_numpy(arr.view(np.int16)).to(device).view(t.bfloat16)
    if dtype_name == "fp8":
        return t.from_numpy(arr).to(device)
    return t.from_numpy(arr.astype(np.float32)).to(device)


def upload(cfg, tensor, device="cuda"):
    """Whole ``tensor`` of ``cfg`` on the device, generated chunk by chunk.
    fp8 indexer tensors return (codes, scale bytes)."""
    t = torch()
    n = cfg.T if tensor in ("q_idx", "w", "q") else cfg.S
    tail = {"q_idx": (cfg.HI, cfg.DI), "k_idx": (cfg.DI,), "w": (cfg.HI,),
            "q": (cfg.H, cfg.D), "kv": (cfg.D,)}[tensor]
    dt = {"q_idx": cfg.idx_dtype, "k_idx": cfg.idx_dtype, "w": cfg.w_dtype,
          "q": cfg.mla_dtype, "kv": cfg.mla_dtype}[tensor]
    tdt = {"bf16": t.bfloat16, "f32": t.float32, "fp8": t.uint8}[dt]
    out = t.empty((cfg.B, n) + tail, dtype=tdt, device=device)
    sf = None
    if dt == "fp8":
        sf = t.empty((cfg.B, n) + tail[:-1] + (cfg.DI // 128,), dtype=t.uint8, device=device)
    for b, r0, r1, stored in iter_blocks(cfg, tensor):
        if dt == "fp8":
            out[b, r0:r1] = to_dev(stored[0], "fp8", device)
            sf[b, r0:r1] = to_dev(stored[1], "fp8", device)
        else:
            out[b, r0:r1] = to_dev(stored, dt, device)
    return (out, sf) if dt == "fp8" else out


def upload_all(cfg, device="cuda"):
    """Every input of the hot path on the device, keyed by tensor name, with
    the fp8 scale bytes under q_sf / k_sf (None for other dtypes)."""
    d = {n: upload(cfg, n, device) for n in ("q_idx", "k_idx", "w", "q", "kv")}
    if cfg.idx_dtype == "fp8":
        d["q_idx"], d["q_sf"] = d["q_idx"]
        d["k_idx"], d["k_sf"] = d["k_idx"]
    else:
        d["q_sf"] = d["k_sf"] = None
    return d


def dev_to_np(x, dtype_name):
    t = torch()
    x = x.detach().cpu().contiguous()
    if dtype_name == "bf16":
        return x.view(t.int16).numpy().view(np.uint16)
    return x.numpy()

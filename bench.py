"""Benchmark of the sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_8k]

A step is one dsa_forward over one batch of the workload (index scores ->
top-2048 -> sparse latent attention), inputs resident in HBM.  The default
workload is the V3.2-shape bf16 decode: batch 32, one query per sequence,
8192 keys, 64x128 indexer heads, 128 MLA heads over 512 + 64.  Inputs rotate
over several device copies so that the 256 MB last-level cache cannot serve
them between steps.

Prints one JSON line: throughput (queries/s), the roofline of the dominant
kernel (timed with HIP events on the stream it runs on), and the CPU oracle's
throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_8k")
    ap.add_argument("--replicas", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample size (0 = auto)")
    ap.add_argument("--only", default="", help="profile one entry point only: forward|indexer|topk|mla")
    return ap.parse_args()


def algorithmic(cfg):
    """Bytes each query must move and flops it must do (inputs read once,
    outputs written once; scores and indices are intermediates)."""
    e = {"bf16": 2, "f32": 4, "fp8": 1}
    ib, wb, mb = e[cfg.idx_dtype], e[cfg.w_dtype], e[cfg.mla_dtype]
    causal_keys = cfg.S if cfg.T == 1 else (cfg.S - cfg.T) + (cfg.T + 1) / 2.0  # mean visible keys
    sel = min(cfg.K_eff, causal_keys)
    nblk = cfg.DI // 128 if cfg.idx_dtype == "fp8" else 0
    idx_bytes = (cfg.S * cfg.DI * ib + cfg.S * nblk) / cfg.T + cfg.HI * cfg.DI * ib + cfg.HI * nblk + cfg.HI * wb
    mla_bytes = sel * cfg.D * mb + cfg.H * cfg.D * mb + cfg.H * cfg.Dc * mb
    if cfg.T > 1:  # prefill: the cache is read once per sequence, not per query
        mla_bytes = cfg.S * cfg.D * mb / cfg.T + cfg.H * cfg.D * mb + cfg.H * cfg.Dc * mb
    idx_flops = 2.0 * cfg.HI * cfg.DI * causal_keys
    mla_flops = 2.0 * cfg.H * (cfg.D + cfg.Dc) * sel
    return dict(indexer_bytes=idx_bytes, mla_bytes=mla_bytes, bytes=idx_bytes + mla_bytes,
                indexer_flops=idx_flops, mla_flops=mla_flops, flops=idx_flops + mla_flops)


def source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "sparse_latent_attention_lightning_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def counters_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        ent = d.get(workload, {}).get(kernel)
        if ent and ent.get("source_hash") == source_hash():
            return ent["hbm_bytes_per_launch"]
    except (ValueError, KeyError):
        return None
    return None


def cpu_baseline(cfg, rows):
    """The oracle (scores -> top-K -> sparse MLA) on `rows` queries of the
    workload, all host cores."""
    import numpy as np

    import dsa_inputs as g
    import oracle
    oracle.build(force=False)
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    all_rows = [(b, t) for b in range(cfg.B) for t in range(cfg.T)]
    pick = sorted(rng.choice(len(all_rows), size=min(rows, len(all_rows)), replace=False))
    rb = np.array([all_rows[i][0] for i in pick], np.int32)
    rt = np.array([all_rows[i][1] for i in pick], np.int32)
    # inputs for the sampled rows (generation is not timed)
    k_idx = {}
    kv = {}
    for b in sorted(set(rb.tolist())):
        k_idx[b] = g.rows(cfg, "k_idx", b, 0, cfg.S)
        kv[b] = g.rows(cfg, "kv", b, 0, cfg.S)
    qi = [g.rows(cfg, "q_idx", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)]
    w = np.concatenate([g.rows(cfg, "w", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)])
    q = np.concatenate([g.rows(cfg, "q", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)])
    t0 = time.perf_counter()
    n = 0
    for b in sorted(set(rb.tolist())):
        sel = rb == b
        sub = cfg.replace(B=1)
        zeros = np.zeros(sel.sum(), np.int32)
        if cfg.idx_dtype == "fp8":
            qc = np.concatenate([qi[i][0] for i in np.nonzero(sel)[0]])
            qs = np.concatenate([qi[i][1] for i in np.nonzero(sel)[0]])
            sc = oracle.indexer_scores(sub, zeros, rt[sel], qc, w[sel], k_idx[b][0][None], qs,
                                       k_idx[b][1][None], threads=threads)
        else:
            qc = np.concatenate([qi[i] for i in np.nonzero(sel)[0]])
            sc = oracle.indexer_scores(sub, zeros, rt[sel], qc, w[sel], k_idx[b][None], threads=threads)
        idx = oracle.topk(sub, sc, threads=threads)
        oracle.sparse_mla(sub, zeros, q[sel], kv[b][None], idx, threads=threads)
        n += int(sel.sum())
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="queries/s", cores=threads, kind="oracle",
                sample=f"{n} of {cfg.B * cfg.T} queries of the workload, full hot path "
                       f"(scores, top-{cfg.K_eff}, sparse MLA) in fp64, {dt:.1f} s wall")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    import dsa_inputs as g
    import sparse_latent_attention_lightning_amd as dsa
    from tests import gpu_util as U

    cfg = g.CONFIGS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    shape = U.shape_of(cfg)
    print(f"[bench] workload {cfg.name}: {cfg}", file=sys.stderr, flush=True)

    base = {n: U.upload(cfg, n, dev) for n in ("q_idx", "k_idx", "w", "q", "kv")}
    if cfg.idx_dtype == "fp8":
        base["q_idx"], base["q_sf"] = base["q_idx"]
        base["k_idx"], base["k_sf"] = base["k_idx"]
    else:
        base["q_sf"] = base["k_sf"] = None
    per_rep = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    reps = args.replicas or max(2, min(8, int(1.0e9 // per_rep) + 1))
    replicas = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                         for _ in range(reps - 1)]
    print(f"[bench] {reps} input copies of {per_rep / 1e6:.0f} MB rotate through the timed loop",
          file=sys.stderr, flush=True)

    ws = torch.zeros(dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD), dtype=torch.uint8, device=dev)
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dc), dtype=base["q"].dtype, device=dev)
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.B, cfg.T, cfg.K_eff), dtype=torch.int32, device=dev)
    scores = torch.empty((cfg.B, cfg.T, cfg.S), dtype=torch.float32, device=dev)
    ws_topk = torch.zeros(max(1, dsa.workspace_bytes(shape, dsa.ENTRY_TOPK)), dtype=torch.uint8, device=dev)
    ws_mla = torch.zeros(max(1, dsa.workspace_bytes(shape, dsa.ENTRY_SPARSE_MLA)), dtype=torch.uint8, device=dev)

    def step(i):
        x = replicas[i % reps]
        dsa.dsa_forward(shape, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["q_sf"], x["k_sf"],
                        ws=ws, out=o, idx_out=idx, lse=lse)

    def run_indexer(i):
        x = replicas[i % reps]
        dsa.dsa_indexer_scores(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"], out=scores)

    def run_topk(i):
        dsa.dsa_topk(shape, scores, out=idx, ws=ws_topk)

    def run_mla(i):
        x = replicas[i % reps]
        dsa.dsa_sparse_mla_fwd(shape, x["q"], x["kv"], idx, out=o, lse=lse, ws=ws_mla)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(warm + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms

    if args.only:
        fn = {"forward": step, "indexer": run_indexer, "topk": run_topk, "mla": run_mla}[args.only]
        if args.only in ("topk", "mla"):
            run_indexer(0)
            run_topk(0)
        ms = timed(fn, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "ms_per_call": ms}))
        return

    ms = timed(step, args.steps, args.warmup)
    print(f"[bench] forward: {ms * 1e3:.1f} us per step", file=sys.stderr, flush=True)

    # per-entry-point timing (same stream, same rotation)
    run_indexer(0)
    run_topk(0)
    kern = {
        "indexer_mfma": (timed(run_indexer, args.steps, 3), "dsa_indexer_scores"),
        "topk_select": (timed(run_topk, args.steps, 3), "dsa_topk"),
        "sparse_mla": (timed(run_mla, args.steps, 3), "dsa_sparse_mla_fwd"),
    }
    for k, (t, _) in kern.items():
        print(f"[bench] {k}: {t * 1e3:.1f} us per launch", file=sys.stderr, flush=True)

    A = algorithmic(cfg)
    q = cfg.B * cfg.T
    step_s = ms / 1e3
    value = q / step_s
    # the dominant single kernel: the indexer (one launch per entry-point call)
    # or the attention entry point, whichever takes longer
    dom = max(("indexer_mfma", "sparse_mla"), key=lambda k: kern[k][0])
    t_dom = kern[dom][0] / 1e3
    if dom == "indexer_mfma":
        bytes_launch = A["indexer_bytes"] * q
        flops_launch = A["indexer_flops"] * q
    else:
        bytes_launch = A["mla_bytes"] * q
        flops_launch = A["mla_flops"] * q
    decode = cfg.T == 1
    if decode:
        achieved = bytes_launch / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops_launch / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = dom
    roof["entry_point"] = kern[dom][1]
    roof["launch_us"] = round(t_dom * 1e6, 2)
    roof["algorithmic_per_launch"] = round(bytes_launch if decode else flops_launch)
    traffic = counters_for(dom, cfg.name)
    roof["traffic"] = traffic

    result = {
        "metric": "indexer+sparse-MLA queries/sec",
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.mla_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "queries_per_seq": cfg.T, "keys": cfg.S,
                   "index_heads": cfg.HI, "index_dim": cfg.DI, "heads": cfg.H, "latent": cfg.Dc,
                   "rope": cfg.Dr, "topk": cfg.K, "idx_dtype": cfg.idx_dtype},
        "step_hbm_frac": round(A["bytes"] * q / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_tokens_per_s": round(value, 1),
        "kernel_us": {k: round(v[0] * 1e3, 2) for k, v in kern.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or (cfg.B * cfg.T if cfg.T == 1 else 16)
        print(f"[bench] CPU oracle on {rows} queries ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, rows)
    print(json.dumps(result))


if __name__ == "__main__":
    main()

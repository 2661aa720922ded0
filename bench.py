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
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    help="all (the four V3.2 workloads; decode_8k is the headline) or one workload")
    ap.add_argument("--replicas", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample size (0 = auto)")
    ap.add_argument("--only", default="", help="profile one entry point only: forward|indexer|topk|mla")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy a MIB-sized device buffer 5 times (the known-size "
                         "kernel the HBM counters are scaled by)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "`--only forward --copy-calibration MIB` into profiles/hbm_counters.json")
    ap.add_argument("--calibration-mib", type=int, default=256)
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("COUNTER_DIR", "UTIL_DIR"),
                    help="no GPU: MFMA work per kernel from a rocprofv3 --pmc run of "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_VALU_MFMA_BUSY_CYCLES "
                         "GRBM_GUI_ACTIVE and one of MfmaUtil")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="no GPU: the kernel table of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-stalls", metavar="DIR",
                    help="no GPU: wave-cycle shares per kernel from a rocprofv3 --pmc run of "
                         "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
                         "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_INSTS_LDS")
    return ap.parse_args()


def algorithmic(cfg):
    """Bytes each query must move and flops it must do, averaged over the
    workload's queries (inputs read once, outputs written once; scores and
    indices are intermediates).  Query t of a sequence sees the keys
    s <= q_pos(t) = S - T + t and attends over min(K, q_pos(t) + 1) of them."""
    e = {"bf16": 2, "f32": 4, "fp8": 1}
    ib, wb, mb = e[cfg.idx_dtype], e[cfg.w_dtype], e[cfg.mla_dtype]
    vis = [cfg.S - cfg.T + t + 1 for t in range(cfg.T)]
    causal_keys = sum(vis) / cfg.T                          # mean visible keys
    sel = sum(min(cfg.K_eff, v) for v in vis) / cfg.T       # mean selected keys
    nblk = cfg.DI // 128 if cfg.idx_dtype == "fp8" else 0
    idx_bytes = (cfg.S * cfg.DI * ib + cfg.S * nblk) / cfg.T + cfg.HI * cfg.DI * ib + cfg.HI * nblk + cfg.HI * wb
    mla_bytes = sel * cfg.D * mb + cfg.H * cfg.D * mb + cfg.H * cfg.Dc * mb
    if cfg.T > 1:  # prefill: the cache is read once per sequence, not per query
        mla_bytes = cfg.S * cfg.D * mb / cfg.T + cfg.H * cfg.D * mb + cfg.H * cfg.Dc * mb
    idx_flops = 2.0 * cfg.HI * cfg.DI * causal_keys
    mla_flops = 2.0 * cfg.H * (cfg.D + cfg.Dc) * sel
    return dict(indexer_bytes=idx_bytes, mla_bytes=mla_bytes, bytes=idx_bytes + mla_bytes,
                indexer_flops=idx_flops, mla_flops=mla_flops, flops=idx_flops + mla_flops)


def roofline(decode, nbytes, nflops, seconds, peak_tflops=MFMA_BF16_PEAK_TFLOPS):
    """HBM roofline (decode) or MFMA roofline (prefill) against the peak of
    the contraction's dtype."""
    if decode:
        achieved = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = nflops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tflops,
            "unit": "TFLOP/s", "frac": round(achieved / peak_tflops, 4)}


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


def _kernel_short_name(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].split("<")[0].split("::")[-1].strip()


def _kernel_template_name(name):
    """Kernel name with its template arguments, without namespaces and the
    parameter list (rocprofv3 without -T reports the full signature)."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("dsa::", "")
    return name.split("(")[0].strip()


def _pmc_rows(d, counter):
    """{kernel: {dispatch id: counter value summed over its instances}}."""
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = per.setdefault(_kernel_short_name(r["Kernel_Name"]), {})
            k[int(r["Dispatch_Id"])] = k.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return per


def summarize_pmc(fetch_dir, write_dir, mib, workload, out_path=None):
    """HBM bytes per launch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the counter reads for the calibration copy
    (the last 5 device-copy dispatches of the run, `mib` MiB each)."""
    fetch = _pmc_rows(fetch_dir, "FETCH_SIZE")
    write = _pmc_rows(write_dir, "WRITE_SIZE")
    ck = "__amd_rocclr_copyBuffer"
    if ck not in fetch or ck not in write:
        raise SystemExit("no copy kernel in the counter runs (run with --copy-calibration)")

    def calib(per):
        last = sorted(per[ck])[-5:]
        return sum(per[ck][i] for i in last) / len(last)

    known_kib = mib * 1024.0
    cf, cw = calib(fetch), calib(write)
    f_fetch, f_write = known_kib / cf, known_kib / cw
    out = {}
    lines = ["| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
             "|---|---|---|---|---|"]
    for k in sorted(fetch):
        if k not in write or k == ck or not k:
            continue
        fv = sum(fetch[k].values()) / len(fetch[k])
        wv = sum(write[k].values()) / len(write[k])
        hbm = (fv * f_fetch + wv * f_write) * 1024.0
        out[k] = {"fetch_kib": round(fv, 1), "write_kib": round(wv, 1),
                  "hbm_bytes_per_launch": round(hbm), "source_hash": source_hash()}
        lines.append(f"| {k} | {len(fetch[k])} | {fv:,.0f} | {wv:,.0f} | {hbm:,.0f} |")
    p = out_path or os.path.join(ROOT, "profiles", "hbm_counters.json")
    d = json.load(open(p)) if os.path.exists(p) else {}
    d[workload] = out
    d[workload]["_calibration"] = {"copy_kernel": ck, "copy_mib": mib, "fetch_kib": round(cf, 1),
                                   "write_kib": round(cw, 1), "fetch_factor": round(f_fetch, 4),
                                   "write_factor": round(f_write, 4)}
    os.makedirs(os.path.dirname(p), exist_ok=True)
    json.dump(d, open(p, "w"), indent=1, sort_keys=True)
    print(f"calibration: {ck} copying {mib} MiB (last 5 dispatches) reads FETCH_SIZE {cf:,.0f} KiB "
          f"and WRITE_SIZE {cw:,.0f} KiB: factors {f_fetch:.4f} (fetch), {f_write:.4f} (write)\n")
    print("\n".join(lines))


def summarize_stalls(d):
    """Per kernel, each SQ counter of the run as a share of the waves' cycles
    (SQ_WAVE_CYCLES: cycles summed over the kernel's resident waves), plus
    the LDS instructions per dispatch; values are the mean over dispatches."""
    shares = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
              "SQ_ACTIVE_INST_LDS")
    base = _pmc_rows(d, "SQ_WAVE_CYCLES")
    cols = {c: _pmc_rows(d, c) for c in shares + ("SQ_INSTS_LDS", "SQ_BUSY_CYCLES")}
    lines = ["| kernel | dispatches | wave cycles | " + " | ".join(c[3:].lower() for c in shares) + " | LDS instructions |",
             "|---|---|---|" + "---|" * len(shares) + "---|"]
    for k in sorted(base):
        if not k or k.startswith("__amd") or "elementwise" in k:
            continue
        n = len(base[k])
        wc = sum(base[k].values()) / n
        row = [k, str(n), f"{wc:,.0f}"]
        for c in shares:
            v = cols[c].get(k)
            row.append(f"{100.0 * sum(v.values()) / n / wc:.1f} %" if v and wc else "—")
        v = cols["SQ_INSTS_LDS"].get(k)
        row.append(f"{sum(v.values()) / n:,.0f}" if v else "—")
        lines.append("| " + " | ".join(row) + " |")
    print("\n".join(lines))


def summarize_trace(d):
    """Markdown table of a rocprofv3 --stats kernel summary (*kernel_stats.csv)."""
    import csv
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    print("| kernel | calls | average us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| {_kernel_template_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")


def summarize_mfma(counter_dir, util_dir):
    """Per kernel: MFMA flops per dispatch (MOPS x 512, bf16 and fp8), the
    dispatch's duration under counter collection, the flop rate that gives,
    and rocprofv3's MfmaUtil (MFMA busy cycles over GPU-active cycles of all
    SIMDs) from a second run."""
    import csv

    def read(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        per = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                k = per.setdefault(_kernel_template_name(r["Kernel_Name"]), {})
                e = k.setdefault(int(r["Dispatch_Id"]), {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return per

    cnt, util = read(counter_dir), read(util_dir)
    print("| kernel | dispatches | bf16 MFMA flops | fp8 MFMA flops | us (counting) | MFMA TFLOP/s | MfmaUtil |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(cnt, key=lambda k: -sum(e["ns"] for e in cnt[k].values())):
        ds = list(cnt[k].values())
        n = len(ds)
        bf = sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for e in ds) / n * 512
        f8 = sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) for e in ds) / n * 512
        us = sum(e["ns"] for e in ds) / n / 1e3
        if bf + f8 == 0:
            continue
        u = [e.get("MfmaUtil") for e in util.get(k, {}).values() if "MfmaUtil" in e]
        util_txt = f"{sum(u) / len(u):.1f} %" if u else "n/a"
        print(f"| {k} | {n} | {bf:.4g} | {f8:.4g} | {us:.1f} | {(bf + f8) / us / 1e6:.1f} | {util_txt} |")


def cpu_model():
    """The host CPU's model name (first /proc/cpuinfo entry)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, rows):
    """The oracle (scores -> top-K -> sparse MLA) on `rows` queries of the
    workload, all host cores: the sampled sequences run side by side on a
    pool of host threads (the oracle's C routines release the GIL), and the
    threads left over split each sequence's query rows."""
    from concurrent.futures import ThreadPoolExecutor

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
    seqs = sorted(set(rb.tolist()))
    outer = max(1, min(threads, len(seqs)))
    inner = max(1, threads // outer)
    # inputs for the sampled rows (generation is not timed)
    k_idx = {}
    kv = {}
    for b in seqs:
        k_idx[b] = g.rows(cfg, "k_idx", b, 0, cfg.S)
        kv[b] = g.rows(cfg, "kv", b, 0, cfg.S)
    qi = [g.rows(cfg, "q_idx", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)]
    w = np.concatenate([g.rows(cfg, "w", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)])
    q = np.concatenate([g.rows(cfg, "q", int(b), int(t), int(t) + 1) for b, t in zip(rb, rt)])
    sub = cfg.replace(B=1)

    def one_sequence(b):
        sel = rb == b
        zeros = np.zeros(sel.sum(), np.int32)
        if cfg.idx_dtype == "fp8":
            qc = np.concatenate([qi[i][0] for i in np.nonzero(sel)[0]])
            qs = np.concatenate([qi[i][1] for i in np.nonzero(sel)[0]])
            sc = oracle.indexer_scores(sub, zeros, rt[sel], qc, w[sel], k_idx[b][0][None], qs,
                                       k_idx[b][1][None], threads=inner)
        else:
            qc = np.concatenate([qi[i] for i in np.nonzero(sel)[0]])
            sc = oracle.indexer_scores(sub, zeros, rt[sel], qc, w[sel], k_idx[b][None], threads=inner)
        idx = oracle.topk(sub, sc, threads=inner)
        oracle.sparse_mla(sub, zeros, q[sel], kv[b][None], idx, threads=inner)
        return int(sel.sum())

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=outer) as ex:
        n = sum(ex.map(one_sequence, seqs))
    dt = time.perf_counter() - t0
    used = min(threads, outer * min(inner, max(int((rb == b).sum()) for b in seqs)))
    return dict(value=n / dt, unit="queries/s", cores=used, cpu=cpu_model(), kind="oracle",
                sample=f"{n} of {cfg.B * cfg.T} queries of the workload from {len(seqs)} sequence(s), "
                       f"full hot path (scores, top-{cfg.K_eff}, sparse MLA) in fp64, {outer} sequence(s) at "
                       f"a time x {inner} thread(s) each, {dt:.1f} s wall")


# The cache fill and indexer inputs of new tokens (the step before the
# path): the joint projection of the V3.2 width (D = 7168 -> 768 outputs)
# plus norms, rotation, E4M3 keys and the scatter into the caches.
FILL_WORKLOADS = {"cache_fill_decode": 32, "cache_fill_prefill": 16384,
                  "indexer_query_decode": 32, "indexer_query_prefill": 16384}
FILL_D = 7168
QUERY_D = 1536   # the query latent width (q_lora_rank)


def bench_cache_fill(args):
    import numpy as np
    import torch

    import sparse_latent_attention_lightning_amd as dsa

    N = FILL_WORKLOADS[args.workload]
    query = args.workload.startswith("indexer_query")
    D = QUERY_D if query else FILL_D
    ncols = 8192 if query else 768
    decode = N <= 256
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    w_bytes = ncols * D * 2
    # rotate over enough weight copies that the 256 MB last-level cache cannot serve them
    reps = args.replicas or (max(2, -(-600_000_000 // (w_bytes + N * D * 2))) if decode else 2)
    xs = [torch.randn((N, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(reps)]
    Ws = [(torch.randn((ncols, D), generator=gen, device=dev) / D ** 0.5).to(torch.bfloat16)
          for _ in range(reps)]
    ones512 = torch.ones(512, device=dev)
    ones128 = torch.ones(128, device=dev)
    zeros128 = torch.zeros(128, device=dev)
    ang = torch.rand((N, 32), generator=gen, device=dev) * 6.283
    cos, sin = torch.cos(ang), torch.sin(ang)
    rows = N
    slots = torch.arange(N, dtype=torch.int64, device=dev)
    kv_cache = torch.empty((rows, 576), dtype=torch.bfloat16, device=dev)
    k_cache = torch.empty((rows, 128), dtype=torch.uint8, device=dev)
    k_sf = torch.empty((rows,), dtype=torch.uint8, device=dev)
    w_out = torch.empty((N, 64), dtype=torch.bfloat16, device=dev)
    if query:
        ws = torch.empty(max(1, dsa.lib().dsa_indexer_query_workspace_bytes(N, D)), dtype=torch.uint8,
                         device=dev)
        q_out = torch.empty((N, 64, 128), dtype=torch.uint8, device=dev)
        q_sf = torch.empty((N, 64), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(max(1, dsa.lib().dsa_cache_fill_workspace_bytes(N, D)), dtype=torch.uint8,
                         device=dev)

    def step(i):
        if query:
            dsa.dsa_indexer_query(xs[i % reps], Ws[i % reps], q_dtype=torch.uint8, q_out=q_out, q_sf=q_sf,
                                  ws=ws)
        else:
            dsa.dsa_cache_fill(xs[i % reps], Ws[i % reps], ones512, ones128, zeros128, cos, sin, slots,
                               kv_cache, k_cache, k_sf, w_out=w_out, ws=ws)

    def timed(n, warm):
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            step(warm + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(args.steps, args.warmup)
    dsa.dsa_timing_begin()
    timed(args.steps, 0)
    kt = dsa.dsa_timing_end()
    for k, r in kt.items():
        print(f"[bench] {k}: {r['avg_us']:.2f} us per launch ({r['launches']} launches)",
              file=sys.stderr, flush=True)
    # algorithmic: the weights and hidden states once, the cache rows, keys,
    # scales and head weights written once
    if query:
        nbytes = w_bytes + N * D * 2 + N * 64 * (128 + 1)
    else:
        nbytes = w_bytes + N * D * 2 + N * (576 * 2 + 128 + 1 + 64 * 2)
    nflops = 2.0 * N * ncols * D
    gemm = "q_gemm" if query else "fill_gemm"
    t_gemm = kt[gemm]["avg_us"] / 1e6
    roof = roofline(decode, nbytes if decode else 0, nflops, t_gemm)
    roof["kernel"] = gemm
    roof["launch_us"] = round(t_gemm * 1e6, 2)
    roof["algorithmic_per_launch"] = round(nbytes if decode else nflops)
    roof["traffic"] = None
    result = {
        "metric": ("indexer-query" if query else "cache-fill") + " tokens/sec",
        "value": round(N / (ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": N, "hidden": D, "outputs": ncols,
                   "out_dtype": "fp8" if query else "kv bf16, k fp8"},
        "kernel_us": {k: round(r["avg_us"], 2) for k, r in kt.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline and not query:
        import oracle
        n_cpu = min(N, 32)
        xb = xs[0][:n_cpu].view(torch.int16).cpu().numpy().view(np.uint16)
        Wb = Ws[0].view(torch.int16).cpu().numpy().view(np.uint16)
        threads = oracle.default_threads()
        t0 = time.perf_counter()
        oracle.cache_fill(xb, Wb, np.ones(512), np.ones(128), np.zeros(128),
                          cos[:n_cpu].cpu().numpy(), sin[:n_cpu].cpu().numpy(), threads=threads)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(n_cpu / dt, 2), "unit": "tokens/s", "cores": threads,
                                  "cpu": cpu_model(), "kind": "oracle",
                                  "sample": f"{n_cpu} tokens of the workload, fp64, {dt:.1f} s wall"}
    print(json.dumps(result))


ABSORB_WORKLOADS = {"absorb_decode": 32, "absorb_prefill": 16384,
                    "wo_decode": 32, "wo_prefill": 16384}
HEADS, WO_IN, WO_OUT = 128, 16384, 7168


def bench_absorb(args):
    """The absorption products either side of the sparse attention: per-head
    W_UK (query) and W_UV (output) products of the 128 heads (absorb_*), or
    the output projection wo 16384 -> 7168 (wo_*), over N tokens."""
    import numpy as np
    import torch

    import sparse_latent_attention_lightning_amd as dsa

    N = ABSORB_WORKLOADS[args.workload]
    wo = args.workload.startswith("wo")
    decode = N <= 256
    H = HEADS
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    rnd = lambda shape, sc=1.0: (torch.randn(shape, generator=gen, device=dev) * sc).to(torch.bfloat16)
    w_bytes = WO_OUT * WO_IN * 2 if wo else H * 256 * 512 * 2 + H * 512 * 128 * 2
    reps = args.replicas or (max(2, -(-600_000_000 // w_bytes)) if decode else 1)
    if wo:
        xs = [rnd((N, WO_IN))]
        Ws = [rnd((WO_OUT, WO_IN), WO_IN ** -0.5) for _ in range(reps)]
        out = torch.empty((N, WO_OUT), dtype=torch.bfloat16, device=dev)
        nb = dsa.lib().dsa_output_projection_workspace_bytes(N, WO_IN, WO_OUT)
        ws = torch.empty(max(1, nb), dtype=torch.uint8, device=dev)
    else:
        qb = rnd((N, H, 192))
        o_lat = rnd((N, H, 512), 0.1)
        kvbs = [rnd((H * 256, 512), 512 ** -0.5) for _ in range(reps)]
        wuks = [dsa.dsa_absorb_prepare(k) for k in kvbs]
        ang = torch.rand((N, 32), generator=gen, device=dev) * 6.283
        cos, sin = torch.cos(ang), torch.sin(ang)
        q = torch.empty((N, H, 576), dtype=torch.bfloat16, device=dev)
        premix = torch.empty((N, H * 128), dtype=torch.bfloat16, device=dev)

    def step(i):
        if wo:
            dsa.dsa_output_projection(xs[0], Ws[i % reps], out=out, ws=ws)
        else:
            dsa.dsa_absorb_query(qb, wuks[i % reps], cos, sin, q=q)
            dsa.dsa_absorb_output(o_lat, kvbs[i % reps], out=premix)

    def timed(n, warm):
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            step(warm + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(args.steps, args.warmup)
    dsa.dsa_timing_begin()
    timed(args.steps, 0)
    kt = dsa.dsa_timing_end()
    for k, r in kt.items():
        print(f"[bench] {k}: {r['avg_us']:.2f} us per launch ({r['launches']} launches)",
              file=sys.stderr, flush=True)
    # algorithmic per launch of the dominant product: its weights once, its
    # inputs once, its outputs written once
    if wo:
        gemm = "wo_gemm"
        nbytes = WO_OUT * WO_IN * 2 + N * WO_IN * 2 + N * WO_OUT * 2
        nflops = 2.0 * N * WO_IN * WO_OUT
    else:
        gemm = "absorb_q_gemm"   # W_UK [128, 512] per head; q^C in, the 512 latent dims out
        nbytes = H * 128 * 512 * 2 + N * H * 128 * 2 + N * H * 512 * 2
        nflops = 2.0 * N * H * 128 * 512
    t_gemm = kt[gemm]["avg_us"] / 1e6
    roof = roofline(decode, nbytes if decode else 0, nflops, t_gemm)
    roof["kernel"] = gemm
    roof["launch_us"] = round(t_gemm * 1e6, 2)
    roof["algorithmic_per_launch"] = round(nbytes if decode else nflops)
    roof["traffic"] = None
    result = {
        "metric": ("output-projection" if wo else "absorption (query + output)") + " tokens/sec",
        "value": round(N / (ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": ({"workload": args.workload, "tokens": N, "in": WO_IN, "out": WO_OUT} if wo else
                   {"workload": args.workload, "tokens": N, "heads": H, "latent": 512,
                    "key_dims": 128, "value_dims": 128}),
        "kernel_us": {k: round(r["avg_us"], 2) for k, r in kt.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        n_cpu = min(N, 8 if wo else 32)
        bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        if wo:
            oracle.linear_bf16(bits(xs[0][:n_cpu]), bits(Ws[0]), threads=threads)
        else:
            kv = kvbs[0].float().cpu().numpy()
            oracle.absorb_query(qb[:n_cpu].float().cpu().numpy(), kv, cos[:n_cpu].double().cpu().numpy(),
                                sin[:n_cpu].double().cpu().numpy(), threads=threads)
            oracle.absorb_output(o_lat[:n_cpu].float().cpu().numpy(), kv, threads=threads)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(n_cpu / dt, 2), "unit": "tokens/s", "cores": threads,
                                  "cpu": cpu_model(), "kind": "oracle",
                                  "sample": f"{n_cpu} tokens of the workload, fp64, {dt:.1f} s wall"}
    print(json.dumps(result))


PATH_WORKLOADS = ("decode_8k", "prefill_16k", "decode_128k", "decode_64k_fp8", "prefill_16k_fp8")


def bench_path(cfg, args, steps, warmup, cpu):
    """One workload of the hot path: `steps` timed dsa_forward calls after
    `warmup` untimed ones, then the same steps with per-launch kernel timing,
    and (cpu) the oracle on a bounded sample.  Returns the record."""
    import torch

    import sparse_latent_attention_lightning_amd as dsa
    from dsa_inputs import device as U

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    shape = U.shape_of(cfg)
    print(f"[bench] workload {cfg.name}: {cfg}", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    base = U.upload_all(cfg, dev)
    per_rep = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    reps = args.replicas or max(2, min(8, int(1.0e9 // per_rep) + 1))
    replicas = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                         for _ in range(reps - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {reps} input copies of {per_rep / 1e6:.0f} MB rotate through the timed loop "
          f"(drawn in {time.perf_counter() - t_gen:.1f} s)", file=sys.stderr, flush=True)

    ws = torch.zeros(dsa.workspace_bytes(shape, dsa.ENTRY_FORWARD), dtype=torch.uint8, device=dev)
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dc), dtype=base["q"].dtype, device=dev)
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.B, cfg.T, cfg.K_eff), dtype=torch.int32, device=dev)

    def step(i):
        x = replicas[i % reps]
        dsa.dsa_forward(shape, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["q_sf"], x["k_sf"],
                        ws=ws, out=o, idx_out=idx, lse=lse)

    def run_indexer(i):
        x = replicas[i % reps]
        dsa.dsa_indexer_scores(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"], out=run_indexer.scores)

    def run_topk(i):
        dsa.dsa_topk(shape, run_indexer.scores, out=idx, ws=run_topk.ws)

    def run_mla(i):
        x = replicas[i % reps]
        dsa.dsa_sparse_mla_fwd(shape, x["q"], x["kv"], idx, out=o, lse=lse, ws=run_mla.ws)

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
        if args.only in ("indexer", "topk", "mla"):
            run_indexer.scores = torch.empty((cfg.B, cfg.T, cfg.S), dtype=torch.float32, device=dev)
            run_topk.ws = torch.zeros(max(1, dsa.workspace_bytes(shape, dsa.ENTRY_TOPK)), dtype=torch.uint8,
                                      device=dev)
            run_mla.ws = torch.zeros(max(1, dsa.workspace_bytes(shape, dsa.ENTRY_SPARSE_MLA)),
                                     dtype=torch.uint8, device=dev)
        fn = {"forward": step, "indexer": run_indexer, "topk": run_topk, "mla": run_mla}[args.only]
        if args.only in ("topk", "mla"):
            run_indexer(0)
            run_topk(0)
        ms = timed(fn, steps, warmup)
        return {"only": args.only, "workload": cfg.name, "ms_per_call": ms}

    ms = timed(step, steps, warmup)
    print(f"[bench] {cfg.name} forward: {ms * 1e3:.1f} us per step", file=sys.stderr, flush=True)

    # The same steps once more with the library's kernel timing on: HIP
    # events around each kernel launch, recorded on the stream it runs on.
    dsa.dsa_timing_begin()
    ms_timed = timed(step, steps, 0)
    kt = dsa.dsa_timing_end()
    for k, r in kt.items():
        print(f"[bench] {cfg.name} {k}: {r['avg_us']:.2f} us per launch ({r['launches']} launches)",
              file=sys.stderr, flush=True)

    A = algorithmic(cfg)
    q = cfg.B * cfg.T
    step_s = ms / 1e3
    value = q / step_s
    decode = cfg.T == 1
    # the dominant kernel: the longest average launch of the step among the
    # kernels that do the path's arithmetic (index scores, attention); the
    # longest launch of all is reported beside it
    modeled = [k for k in kt if k.startswith("indexer") or (k.startswith("mla") and k != "mla_combine")]
    dom = max(modeled, key=lambda k: kt[k]["avg_us"])
    longest = max(kt, key=lambda k: kt[k]["avg_us"])
    t_dom = kt[dom]["avg_us"] / 1e6
    peak = MFMA_BF16_PEAK_TFLOPS
    if dom.startswith("indexer"):
        bytes_launch, flops_launch = A["indexer_bytes"] * q, A["indexer_flops"] * q
        peak = MFMA_FP8_PEAK_TFLOPS if cfg.idx_dtype == "fp8" else MFMA_BF16_PEAK_TFLOPS
    elif dom.startswith("mla") and dom != "mla_combine":
        bytes_launch, flops_launch = A["mla_bytes"] * q, A["mla_flops"] * q
    else:
        raise SystemExit(f"bench: no algorithmic model for dominant kernel {dom}")
    roof = roofline(decode, bytes_launch, flops_launch, t_dom, peak)
    roof["kernel"] = dom
    roof["launch_us"] = round(t_dom * 1e6, 2)
    if longest != dom:
        roof["longest_kernel"] = longest
    roof["algorithmic_per_launch"] = round(bytes_launch if decode else flops_launch)
    roof["traffic"] = counters_for(dom, cfg.name)
    # each stage of the path against its own bound (the attention stage is
    # every mla_* kernel of the step)
    stage_us = {"indexer": sum(r["avg_us"] for k, r in kt.items() if k.startswith("indexer")),
                "topk": sum(r["avg_us"] for k, r in kt.items() if k.startswith("topk")),
                "sparse_mla": sum(r["avg_us"] for k, r in kt.items() if k.startswith("mla"))}
    idx_peak = MFMA_FP8_PEAK_TFLOPS if cfg.idx_dtype == "fp8" else MFMA_BF16_PEAK_TFLOPS
    stages = {
        "indexer": roofline(decode, A["indexer_bytes"] * q, A["indexer_flops"] * q, stage_us["indexer"] / 1e6,
                            idx_peak),
        "sparse_mla": roofline(decode, A["mla_bytes"] * q, A["mla_flops"] * q, stage_us["sparse_mla"] / 1e6),
    }
    for k, v in stages.items():
        v["us"] = round(stage_us[k], 2)
    stages["topk"] = {"us": round(stage_us["topk"], 2), "bound": "alu"}
    rec = {
        "workload": cfg.name,
        "value": round(value, 1),
        "unit": "queries/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "dtype": "bf16" if cfg.mla_dtype == "bf16" else "f32",
        "config": {"workload": cfg.name, "batch": cfg.B, "queries_per_seq": cfg.T, "keys": cfg.S,
                   "index_heads": cfg.HI, "index_dim": cfg.DI, "heads": cfg.H, "latent": cfg.Dc,
                   "rope": cfg.Dr, "topk": cfg.K, "idx_dtype": cfg.idx_dtype},
        "step_roofline": roofline(decode, A["bytes"] * q, A["flops"] * q, step_s),
        "step_tokens_per_s": round(value, 1),
        "kernel_us": {k: round(r["avg_us"], 2) for k, r in kt.items()},
        "ms_per_step_kernel_timing": round(ms_timed, 5),
        "stages": stages,
        "roofline": roof,
    }
    if cfg.T < 8 and cfg.S <= 262144:
        # the fused index scores -> top-K launch against the two launches
        # dsa_forward uses, on the same inputs
        scores = torch.empty((cfg.B, cfg.T, cfg.S), dtype=torch.float32, device=dev)
        ws_tk = torch.zeros(max(1, dsa.workspace_bytes(shape, dsa.ENTRY_TOPK)), dtype=torch.uint8, device=dev)
        ws_it = torch.zeros(dsa.workspace_bytes(shape, dsa.ENTRY_INDEXER_TOPK), dtype=torch.uint8, device=dev)

        def fused(i):
            x = replicas[i % reps]
            dsa.dsa_indexer_topk(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"], out=idx, ws=ws_it)

        def separate(i):
            x = replicas[i % reps]
            dsa.dsa_indexer_scores(shape, x["q_idx"], x["k_idx"], x["w"], x["q_sf"], x["k_sf"], out=scores)
            dsa.dsa_topk(shape, scores, out=idx, ws=ws_tk)

        rec["indexer_topk_us"] = {"fused": round(1e3 * timed(fused, steps, warmup), 2),
                                  "separate": round(1e3 * timed(separate, steps, warmup), 2)}
        print(f"[bench] {cfg.name} index scores + top-K: fused {rec['indexer_topk_us']['fused']} us, "
              f"separate {rec['indexer_topk_us']['separate']} us", file=sys.stderr, flush=True)
        del scores, ws_tk, ws_it
    del replicas, base, ws
    torch.cuda.empty_cache()
    if cpu:
        # a bounded sample of about 1-20 s of host work: decode, every query
        # (e4m3: 16 of them; the oracle decodes e4m3 per element); prefill,
        # 512 query rows (e4m3: 64)
        if cfg.T == 1:
            rows = cfg.B if cfg.idx_dtype != "fp8" else min(cfg.B, 16)
        else:
            rows = 64 if cfg.idx_dtype == "fp8" else 512
        rows = args.cpu_rows or rows
        print(f"[bench] {cfg.name}: CPU oracle on {rows} queries ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, rows)
    return rec


def main():
    args = parse()
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.calibration_mib, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.workload in FILL_WORKLOADS:
        bench_cache_fill(args)
        return
    if args.workload in ABSORB_WORKLOADS:
        bench_absorb(args)
        return
    import dsa_inputs as g

    names = PATH_WORKLOADS if args.workload == "all" else (args.workload,)
    recs = {}
    for n in names:
        cfg = g.CONFIGS[n]
        # prefill steps take milliseconds: fewer of them keep the run short
        steps = args.steps if cfg.T == 1 else max(3, min(args.steps, 10))
        warmup = args.warmup if cfg.T == 1 else max(1, min(args.warmup, 3))
        recs[n] = bench_path(cfg, args, steps, warmup, not args.no_cpu_baseline)
        if args.only:
            print(json.dumps(recs[n]))
            if args.copy_calibration:
                copy_calibration(args.copy_calibration)
    if args.only:
        return
    head = recs[names[0]]
    result = {
        "metric": "indexer+sparse-MLA queries/sec",
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
    }
    for k in ("step_roofline", "step_tokens_per_s", "kernel_us", "ms_per_step_kernel_timing", "stages",
              "indexer_topk_us", "roofline", "cpu_baseline"):
        if k in head:
            result[k] = head[k]
    if len(names) > 1:
        result["workloads"] = {n: recs[n] for n in names[1:]}
    print(json.dumps(result))


def copy_calibration(mib):
    """Copy a `mib`-sized device buffer 5 times: the known-size kernel the
    HBM counters are scaled by."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copied {mib} MiB 5 times", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()

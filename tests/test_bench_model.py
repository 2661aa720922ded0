"""The benchmark's measurement model on the CPU: the algorithmic bytes and
flops of each workload against their closed forms (the units the roofline
prices), the roofline arithmetic, and the counter summaries on small
synthetic rocprofv3 outputs (the calibration scaling, per-dispatch averages,
kernel names with template arguments)."""
import csv
import json
import os

import pytest

import bench
import dsa_inputs as g



def _total(name):
    c = g.CONFIGS[name]
    return {k: v * c.B * c.T for k, v in bench.algorithmic(c).items()}


def test_decode_8k_units():
    A = _total("decode_8k")
    per_query_idx = 8192 * 128 * 2 + 64 * 128 * 2 + 64 * 2      # k^I once, Q^I, w
    per_query_mla = 2048 * 1152 + 128 * 1152 + 128 * 512 * 2    # selected rows, q, o
    assert A["indexer_bytes"] == pytest.approx(32 * per_query_idx, rel=1e-12)
    assert A["mla_bytes"] == pytest.approx(32 * per_query_mla, rel=1e-12)
    assert A["mla_flops"] == pytest.approx(32 * 2 * 128 * (576 + 512) * 2048, rel=1e-12)
    assert A["indexer_flops"] == pytest.approx(32 * 2 * 64 * 128 * 8192, rel=1e-12)


def test_prefill_16k_counts_causal_selection():
    A = _total("prefill_16k")
    pairs = sum(min(2048, t + 1) for t in range(16384))         # 31,458,304 selected (query, key) pairs
    assert pairs == 31_458_304
    assert A["mla_flops"] == pytest.approx(pairs * 128 * 1088 * 2, rel=1e-12)   # 8.762e12
    visible = 16384 * 16385 // 2
    assert A["indexer_flops"] == pytest.approx(visible * 2 * 64 * 128, rel=1e-12)
    # the cache is read once per sequence, not once per query
    mla_bytes = 16384 * 1152 + 16384 * (128 * 1152 + 128 * 1024)
    assert A["mla_bytes"] == pytest.approx(mla_bytes, rel=1e-12)


def test_e4m3_decode_counts_scale_bytes():
    A = _total("decode_64k_fp8")
    per_query = 65536 * 128 + 65536 * 1 + 64 * 128 + 64 * 1 + 64 * 2   # codes, key scales, Q^I codes + scales, w
    assert A["indexer_bytes"] == pytest.approx(64 * per_query, rel=1e-12)


def test_roofline_arithmetic():
    r = bench.roofline(True, 8e9, 0, 1e-3)                    # 8 GB in 1 ms: the HBM peak
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(1.0)
    r = bench.roofline(False, 0, 2.5e12, 1e-3)                 # 2.5 TFLOP in 1 ms: the bf16 peak
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(1.0)
    r = bench.roofline(False, 0, 2.5e12, 1e-3, bench.MFMA_FP8_PEAK_TFLOPS)
    assert r["frac"] == pytest.approx(0.5)


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_hbm_counter_summary_scales_by_the_copy(tmp_path):
    k = "void dsa::(anonymous namespace)::mla_mfma(int, int)"
    fetch = [(1, k, "FETCH_SIZE", 1000.0, 0, 1), (2, k, "FETCH_SIZE", 1200.0, 0, 1)]
    write = [(1, k, "WRITE_SIZE", 300.0, 0, 1), (2, k, "WRITE_SIZE", 500.0, 0, 1)]
    for i in range(5):   # the calibration copy of 4 MiB: FETCH_SIZE sees half of it
        fetch.append((10 + i, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 2048.0, 0, 1))
        write.append((10 + i, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 4096.0, 0, 1))
    _counter_csv(str(tmp_path / "f" / "x_counter_collection.csv"), fetch)
    _counter_csv(str(tmp_path / "w" / "x_counter_collection.csv"), write)
    out = tmp_path / "hbm.json"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), 4, "wl", out_path=str(out))
    d = json.load(open(out))["wl"]
    assert d["_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert d["_calibration"]["write_factor"] == pytest.approx(1.0)
    assert d["mla_mfma"]["hbm_bytes_per_launch"] == round((1100.0 * 2 + 400.0) * 1024)


def test_mfma_counter_summary(tmp_path, capsys):
    k = "void dsa::(anonymous namespace)::indexer_prefill<1>(int, int)"
    rows = [(1, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6, 0, 2000), (1, k, "SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0, 0, 2000),
            (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 5.0, 0, 2000), (1, k, "GRBM_GUI_ACTIVE", 9.0, 0, 2000)]
    _counter_csv(str(tmp_path / "c" / "x_counter_collection.csv"), rows)
    _counter_csv(str(tmp_path / "u" / "x_counter_collection.csv"), [(1, k, "MfmaUtil", 42.0, 0, 2000)])
    bench.summarize_mfma(str(tmp_path / "c"), str(tmp_path / "u"))
    line = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| indexer_prefill<1>")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert float(cells[2]) == pytest.approx(512e6)            # MOPS x 512
    assert float(cells[4]) == pytest.approx(2.0)              # 2000 ns
    assert float(cells[5]) == pytest.approx(512e6 / 2e-6 / 1e12, rel=1e-3)
    assert cells[6] == "42.0 %"


def test_kernel_names():
    assert bench._kernel_template_name(
        "void dsa::(anonymous namespace)::topk_select<8, false, false, true>(int, long, int)") == \
        "topk_select<8, false, false, true>"
    assert bench._kernel_short_name("void dsa::(anonymous namespace)::mla_combine<8>(int)") == "mla_combine"

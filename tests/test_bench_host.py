"""Host logic of bench.py (no GPU): the one-GPU guard, the mode guards, the
algorithmic byte counts and the traffic summary's source check."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--gpus", "8", "--steps", "1"]])
def test_more_than_one_gpu_is_refused(args):
    r = run_bench(*args)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args", [["--accum", "mfma8_pow2"],
                                  ["--workload", "decode_grouped", "--accum", "mfma8_pow2"]])
def test_power_of_two_mode_needs_power_of_two_scales(args):
    r = run_bench(*args)
    assert r.returncode == 2
    assert "power-of-two" in r.stderr


def test_algorithmic_bytes_of_the_quantisers():
    # 2 B read + 1 B written per element, 4 B per 1x128 group or 128x128 block
    assert bench.quant_bytes_row(4096, 7168) == 4096 * 7168 * 3 + 4096 * 56 * 4
    assert round(bench.quant_bytes_row(4096, 7168) / 1e6, 1) == 89.0
    assert bench.quant_bytes_block(18432, 7168) == 18432 * 7168 * 3 + 144 * 56 * 4
    assert round(bench.quant_bytes_block(18432, 7168) / 1e6, 1) == 396.4
    # a ragged last block-row still counts one scale per block
    assert bench.quant_bytes_block(130, 256) == 130 * 256 * 3 + 2 * 2 * 4


def test_traffic_is_used_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    label = bench.DENSE_GEMM_LABEL
    good = tmp_path / "summary.md"
    good.write_text(f"# title: with a colon\nsource_hash: {bench.source_hash(bench.PROFILE_SOURCES)}\n"
                    f"traffic | {label} | 1234\ntraffic | quant_tile X[4096x7168] | 99\n")
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", str(good))
    assert bench.measured_traffic(label) == 1234.0
    assert bench.measured_traffic("quant_tile X[4096x7168]") == 99.0
    assert bench.measured_traffic("some other kernel") is None
    stale = tmp_path / "stale.md"
    stale.write_text(f"source_hash: 0000000000000000\ntraffic | {label} | 1234\n")
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", str(stale))
    assert bench.measured_traffic(label) is None
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", str(tmp_path / "absent.md"))
    assert bench.measured_traffic(label) is None


TRACE_HEAD = "Kind,Agent_Id,Queue_Id,Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
PMC_HEAD = "Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
SPIN = "at::cuda::(anonymous namespace)::spin_kernel(long)"


def _write_pass(path, rows, pmc):
    path.mkdir(parents=True)
    with open(path / ("p_counter_collection.csv" if pmc else "p_kernel_trace.csv"), "w") as f:
        f.write(PMC_HEAD if pmc else TRACE_HEAD)
        for r in rows:
            f.write(",".join(f'"{x}"' if isinstance(x, str) and "," in x else str(x) for x in r) + "\n")


def test_profile_summary_splits_dispatches_at_the_markers(tmp_path, monkeypatch):
    """Two labels, 3 launches each; label A launches one kernel per call,
    label B two (a GEMM and its reduction).  Dispatches before the first
    marker (warm-up) and torch kernels outside the segments are ignored;
    counters are divided per launch and scaled by the copy probe."""
    calls = bench.PROFILE_CALLS
    seq = [("void fp8bs::warm_kernel<1>(fp8bs::GemmArgs)", 999)]  # before the first marker
    seq.append((SPIN, 1))
    seq += [("void fp8bs::quant_row_kernel<false, 4>(int)", 10)] * calls
    seq.append((SPIN, 1))
    seq.append(("void fp8bs::setup_kernel(int)", 777))  # between two kernels' segments: not counted
    seq.append((SPIN, 1))
    seq += [("void fp8bs::gemm_kernel<1, 0, 1, 1, true>(fp8bs::GemmArgs, long, long)", 100),
            ("void fp8bs::splitk_reduce_kernel<1>(float const*)", 20)] * calls
    seq.append((SPIN, 1))
    trace, fetch, write, sq = [], [], [], []
    for i, (name, w) in enumerate(seq):
        did = 100 + i
        trace.append(("KERNEL_DISPATCH", 1, 1, did, name, 1000 * i, 1000 * i + 1000 * w))  # w us
        fetch.append((did, name, 64, "FETCH_SIZE", 2.0 * w))     # KiB, probe factor 2
        write.append((did, name, 64, "WRITE_SIZE", 1.0 * w))
        sq.append((did, name, 64, "GRBM_GUI_ACTIVE", 8 * 2000.0 * w))  # 2 GHz over w us
        sq.append((did, name, 64, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000.0 * w))  # half busy
        sq.append((did, name, 64, "SQ_INSTS_VALU", 0.0))
    root = tmp_path / "prof"
    _write_pass(root / "trace", trace, False)
    _write_pass(root / "fetch", fetch, True)
    _write_pass(root / "write", write, True)
    _write_pass(root / "sq", sq, True)
    gib = float(1 << 30)
    _write_pass(root / "probe_fetch", [(1, "neg_kernel", 64, "FETCH_SIZE", 2 * gib / 1024)], True)
    _write_pass(root / "probe_write", [(1, "neg_kernel", 64, "WRITE_SIZE", gib / 1024)], True)
    man = tmp_path / "manifest.json"
    man.write_text("[bench] log line\n" + json.dumps({"profile_manifest": [
        {"workload": "w", "label": "A", "calls": calls, "work": 20480.0, "unit": "GB/s", "bytes": 20480.0},
        {"workload": "w", "label": "B", "calls": calls, "work": 1.0, "unit": "TFLOP/s", "bytes": None}],
        "source_hash": bench.source_hash(bench.PROFILE_SOURCES)}) + "\n")
    out = tmp_path / "summary.md"
    bench.summarize_profile(str(root), str(man), str(out), ["cmd one", "cmd two"])
    text = out.read_text()
    assert "    cmd one" in text and "`quant_row_kernel<false, 4>`" in text
    assert "`gemm_kernel<1, 0, 1, 1, true>`, `splitk_reduce_kernel<1>`" in text
    got = bench.read_profile_summary(str(out))
    # A: a 20 KiB FETCH_SIZE (probe factor 2: 10 KiB read) + 10 KiB written per launch
    assert got["A"] == pytest.approx(10 * 1024 + 10 * 1024)
    # B: (200 + 40) KiB FETCH_SIZE / 2 + (100 + 20) KiB written per launch
    assert got["B"] == pytest.approx(120 * 1024 + 120 * 1024)
    row_b = next(ln for ln in text.splitlines() if ln.startswith("| w | B |"))
    cells = [c.strip() for c in row_b.split("|")]
    assert cells[4] == "120.0"            # us per launch
    assert cells[9] == "50.0%" and cells[11] == "2.00"  # MFMA busy, clock
    row_a = next(ln for ln in text.splitlines() if ln.startswith("| w | A |"))
    assert row_a.split("|")[7].strip() == "1.00"  # traffic equals the algorithmic bytes


def test_profile_summary_needs_a_marker_per_kernel(tmp_path):
    root = tmp_path / "prof"
    _write_pass(root / "trace", [("KERNEL_DISPATCH", 1, 1, 1, SPIN, 0, 10),
                                 ("KERNEL_DISPATCH", 1, 1, 2, "k", 10, 20),
                                 ("KERNEL_DISPATCH", 1, 1, 3, SPIN, 20, 30)], False)
    with pytest.raises(RuntimeError, match="marker"):
        bench._segments(bench._dispatches(str(root / "trace"), "kernel_trace.csv"), 2)


def _tiny_sample():
    import numpy as np
    import oracle
    from block_scaled_gemm_amd import inputs
    orc = oracle.default()
    d = inputs.tiny_fprop()
    qx, sx = orc.quant_tile(d["X"], 0, 0)
    qw, sw, _ = orc.quant_block(d["W"], 0)
    r = orc.gemm(qx, sx, qw, sw, 0, sw.shape[1], 1)
    y = inputs.bf16_bits(r.astype(np.float32))
    return {"ms": 128, "ns": 256, "qx": qx, "sx": sx, "qw": qw, "sw": sw, "r": r}, y


def test_parity_reports_the_comparator_and_the_codes(monkeypatch):
    """bench.parity on the tiny Fprop: the oracle's own result rounded to
    bf16 passes in every mode; a changed code or a changed output fails."""
    import numpy as np
    monkeypatch.setattr(bench, "K", 512)
    sample, y = _tiny_sample()
    for accum in (0, 1):
        p = bench.parity(sample, y, sample["qx"], sample["sx"], sample["qw"], sample["sw"], accum)
        assert p["gate_passed"] and p["codes_scales_bitexact"], p
        assert p["normwise"] <= 2.0 ** -8 and p["elementwise_within_tol"]
    qx = sample["qx"].copy()
    qx[5, 7] ^= 0x80
    p = bench.parity(sample, y, qx, sample["sx"], sample["qw"], sample["sw"], 1)
    assert not p["codes_scales_bitexact"] and not p["gate_passed"]
    y2 = y.copy()
    y2[3, 4] ^= 0x8000  # flip the sign of one bf16 output
    p = bench.parity(sample, y2, sample["qx"], sample["sx"], sample["qw"], sample["sw"], 1)
    assert p["codes_scales_bitexact"] and not p["gate_passed"]


def test_cpu_quant_baseline_reports_both_thread_counts():
    from block_scaled_gemm_amd import inputs
    d = inputs.tiny_fprop()
    q = bench.cpu_quant_baseline(d["X"], d["W"], reps=1)
    for name in ("quant_tile_row_X", "quant_block_W"):
        assert q[name]["GB/s_1_thread"] > 0 and q[name]["GB/s_all_threads"] > 0
        assert q[name]["threads"] >= 1

"""Host logic of bench.py (no GPU): the one-GPU guard, the mode guards, the
algorithmic byte counts and the traffic summary's source check."""
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
    kernel = bench.GEMM_KERNEL["mfma8"]
    good = tmp_path / "traffic.txt"
    good.write_text(f"# comment: with a colon\nkernel: {kernel}\nsource_hash: {bench.source_hash(bench.KERNEL_SOURCES)}\n"
                    "bytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic(kernel) == 1234.0
    assert bench.measured_traffic("some_other_kernel<0>") is None
    stale = tmp_path / "stale.txt"
    stale.write_text(f"kernel: {kernel}\nsource_hash: 0000000000000000\nbytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic(kernel) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.measured_traffic(kernel) is None


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

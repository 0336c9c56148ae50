"""Benchmark of the fine-grained FP8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-workloads] [--accum mfma8|fp32]
    python bench.py --workload expert_backward|grouped_upproj|decode_grouped|moe_backward
    python bench.py --traffic-probe     # plain copy of known size, for counter scaling
    python bench.py --library-ceiling   # vendor GEMMs on the dense shape, for context

Default line (the headline): the dense Fprop at real width -- X[4096 x 7168]
bf16 ~N(0,1) with 0.1% x100 outliers, W[18432 x 7168] bf16 ~N(0,0.02).  One
step is the whole hot path over that batch, inputs already in HBM:
    quantise X in 1x128 tiles    (fp8_quant_tile, FP32 scales)
    quantise W in 128x128 blocks (fp8_quant_block, FP32 scales)
    Y = X W^T, block-scaled FP8 GEMM with per-128 FP32 promotion, bf16 out.
`value` is the step's GEMM FLOPs over the step time (quantisation
included); `roofline` covers the dominant kernel (the GEMM), its duration
measured with HIP events on the stream it runs on.  Before the warmup steps
each workload's step runs back to back for --settle seconds (untimed; the
count is reported): after an idle gap the shader clock takes ~30-80 ms of
sustained load to settle, and the timed steps measure the settled clock.

The GEMM's accumulation mode is --accum: mfma8 (default) forms each
128-element group partial on the FP8 matrix cores and promotes it in FP32
registers -- the pages' scheme; fp32 forms the partials exactly on the f16
matrix cores.  `parity` compares the timed step's output with the oracle on
the CPU-baseline sample: codes and scales bit for bit, and the GEMM by the
comparator of oracle/compare.py -- normwise max|Y-R|/max|R|, elementwise
max|Y-R|/max(|R|, 1% max|R|), and the error over the FP8-matrix-core bound.
The FP8-matrix-core modes meet the normwise tolerance (8e-3 for bf16) and
the bound on every workload; on some workloads, this one included, their
elementwise figure is above 8e-3 (their limited sum inside each group on
small outputs); the exact mode meets the tolerance on both.  `parity`
reports which.  `gemm_modes` times the dense GEMM in all three modes (the
power-of-two mode on power-of-two quantisations of the same tensors).

`workloads` (skipped with --no-workloads) times the other shapes the path is
measured on, each a step of its own kernels with HIP events:
  expert_backward: dY[8192x2048] quantised both ways in one pass, X's 1x128
    forward codes re-tiled to 128x1, Dgrad 8192x7168x2048 and Wgrad
    2048x7168x8192, fp32 out (W's transposed codes come from the forward);
  grouped_upproj: 32 local experts of a top-8-of-256 routing of 4096 tokens,
    quant X 1x128 + quant W[32x4096x7168] 128x128 (power-of-two scales) +
    grouped GEMM (power-of-two scales inside the MFMA), bf16 out;
  decode_grouped: 64 experts with 1..256 rows, N = 2048, the same steps with
    FP32 scales;
  moe_backward: the up-projection experts' backward pass: dY quantised
    1x128, M-grouped Dgrad on the transposed forward weight codes, dY and X
    quantised in 128x1 groups per expert, K-grouped Wgrad, fp32 out.
--workload NAME prints one such workload as the line instead.

`cpu_baseline` is the CPU oracle on a bounded sub-block of the dense
workload (GEMM) plus its quantisers on 1 thread and on all threads.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 4096, 18432, 7168
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
# per-launch HBM traffic and counters of every workload kernel, written by
# --summarize-profile from the rocprofv3 passes over --profile-kernels
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "kernels_per_launch.md")
PROFILE_SOURCES = ["block_scaled_gemm_amd/csrc/gemm.hip", "block_scaled_gemm_amd/csrc/quant.hip",
                   "block_scaled_gemm_amd/csrc/device.h", "block_scaled_gemm_amd/csrc/kernels.h",
                   "block_scaled_gemm_amd/csrc/api.cpp"]
PROFILE_CALLS = 3
# the dense Fprop GEMM of the default line, as --profile-kernels labels it
DENSE_GEMM_LABEL = "gemm 4096x18432x7168 (FP32 scales, FP8 matrix cores)"
# the kernel one dense-Fprop GEMM call launches, per accumulation mode
GEMM_KERNEL = {"mfma8": "gemm_wide_kernel<1, 0, 0>", "fp32": "gemm_kernel<0, 0, 0, 0, false>"}
METRIC = "block-scaled FP8 GEMM TFLOP/s (% MFMA peak); quantize GB/s (% HBM peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def quant_bytes_row(rows, cols):
    """Algorithmic bytes of 1x128 quantisation: 2 B in, 1 B out per
    element, 4 B per group."""
    return rows * cols * 3 + rows * (cols // 128) * 4


def quant_bytes_block(rows, cols):
    return rows * cols * 3 + ((rows + 127) // 128) * (cols // 128) * 4


def read_profile_summary(path=None):
    """{label: HBM bytes per launch} from the committed summary, or {} when it
    is absent or was taken on other kernel sources.  Machine-readable lines
    of the summary: `source_hash: H` and `traffic | <label> | <bytes>`."""
    try:
        with open(path or PROFILE_SUMMARY) as f:
            lines = f.read().splitlines()
    except OSError:
        return {}
    h = next((ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("source_hash:")), None)
    if h != source_hash(PROFILE_SOURCES):
        return {}
    out = {}
    for ln in lines:
        if ln.startswith("traffic | "):
            _, label, b = [x.strip() for x in ln.split("|")]
            out[label] = float(b)
    return out


def measured_traffic(label):
    """HBM bytes per launch of the workload kernel `label` (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None."""
    return read_profile_summary().get(label)


def traffic_probe():
    """A plain copy of known size (y = -x over 2^28 fp32: 1 GiB read, 1 GiB
    written), launched 3 times, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "torch.neg fp32", "elements": n, "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": 3}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(X, W, target_s=20.0):
    """Time the CPU oracle on a sub-block of the workload: quantise X rows
    [0, ms) and W rows [0, ns), then their GEMM; grow the block until the run
    takes about target_s.  Returns (baseline dict, the sample's oracle
    results for the parity check)."""
    import oracle
    orc = oracle.default()
    ms, ns = 16, 1024
    while True:
        x, w = X[:ms], W[:ns]
        t0 = time.perf_counter()
        qx, sx = orc.quant_tile(x, 0, 0)
        qw, sw, _ = orc.quant_block(w, 0)
        r = orc.gemm(qx, sx, qw, sw, 0, sw.shape[1], 1)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or (ms >= M and ns >= N):
            break
        grow = max(2.0, min(64.0, target_s / max(dt, 1e-3)))
        if ns < N:
            ns = min(N, (int(ns * grow) + 127) // 128 * 128)
        else:
            ms = min(M, int(ms * grow))
    flops = 2.0 * ms * ns * K
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"X rows 0..{ms - 1} x W rows 0..{ns - 1} of the same workload "
                      f"(quant 1x128 + quant 128x128 + GEMM {ms}x{ns}x{K}), {dt:.1f} s",
            "cpu_model": cpu_model()}
    return base, {"ms": ms, "ns": ns, "qx": qx, "sx": sx, "qw": qw, "sw": sw, "r": r}


def cpu_quant_baseline(X, W, reps=5):
    """The oracle's quantisers on a bounded sample of X (rows 0..1023) and
    of W (rows 0..2047), on 1 thread and on all threads, median of `reps`."""
    import oracle
    orc = oracle.default()
    allt = orc.num_threads()
    xs, ws = X[:1024], W[:2048]
    out = {}
    for name, fn, nbytes in (
            ("quant_tile_row_X", lambda: orc.quant_tile(xs, 0, 0), quant_bytes_row(*xs.shape)),
            ("quant_block_W", lambda: orc.quant_block(ws, 0), quant_bytes_block(*ws.shape))):
        row = {"sample": f"{'X' if name.endswith('X') else 'W'}[0:{(xs if name.endswith('X') else ws).shape[0]}] "
                         f"({nbytes / 1e6:.1f} MB)"}
        for label, threads in (("1_thread", 1), ("all_threads", allt)):
            orc.set_num_threads(threads)
            times = []
            for _ in range(reps):
                t0 = time.perf_counter()
                fn()
                times.append(time.perf_counter() - t0)
            row[f"GB/s_{label}"] = nbytes / float(np.median(times)) / 1e9
        row["threads"] = allt
        out[name] = row
    orc.set_num_threads(0)
    return out


def parity(sample, y_bits, qx, sx, qw, sw, accum):
    """The timed step's output and quantisations against the oracle's on
    the CPU-baseline sample (not timed)."""
    import oracle
    orc = oracle.default()
    ms, ns = sample["ms"], sample["ns"]
    codes_ok = (np.array_equal(qx[:ms], sample["qx"]) and np.array_equal(sx[:, :ms], sample["sx"])
                and np.array_equal(qw[:ns], sample["qw"]) and np.array_equal(sw[:(ns + 127) // 128], sample["sw"]))
    sws = sample["sw"]
    rabs = orc.gemm_abs(sample["qx"], sample["sx"], sample["qw"], sws, 0, sws.shape[1], 1)
    y = (np.asarray(y_bits[:ms, :ns], np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = oracle.measure(y, sample["r"], rabs, 0, K // 128)
    ok, why = oracle.passes(m, 0, accum)
    tol = oracle.TOL[0]
    return {"sample": f"Y rows 0..{ms - 1} x columns 0..{ns - 1} (bf16 out)",
            "codes_scales_bitexact": bool(codes_ok),
            "normwise": m["normwise"], "elementwise": m["elementwise"], "bound_ratio": m["bound_ratio"],
            "tol": tol, "normwise_within_tol": m["normwise"] <= tol,
            "elementwise_within_tol": m["elementwise"] <= tol,
            "gate": ("normwise and elementwise <= tol" if accum == 0
                     else "normwise <= tol and error / bound <= 1 (elementwise reported)"),
            "gate_passed": bool(ok and codes_ok), "gate_reason": why if codes_ok else "codes or scales differ"}


def _clock_files():
    """sysfs files of the GPU torch uses: the DPM clock table (its line
    marked '*' is the current shader clock) and the power reading (uW); None
    where absent.  With several cards visible the one on torch's PCI bus is
    taken."""
    import torch
    try:
        props = torch.cuda.get_device_properties(0)
        bus, dom = getattr(props, "pci_bus_id", None), getattr(props, "pci_domain_id", 0) or 0
        cards = sorted(glob.glob("/sys/class/drm/card[0-9]*/device"))
        if bus is not None and len(cards) > 1:
            want = f"{dom:04x}:{bus:02x}:"
            cards = [c for c in cards if os.path.basename(os.path.realpath(c)).startswith(want)] or cards
        if not cards:
            return None, None
        sclk = os.path.join(cards[0], "pp_dpm_sclk")
        power = sorted(glob.glob(os.path.join(cards[0], "hwmon", "hwmon*", "power1_input")))
        return (sclk if os.path.exists(sclk) else None), (power[0] if power else None)
    except Exception:
        return None, None


def _read_sclk_mhz(path):
    with open(path) as f:
        for line in f:
            if line.rstrip().endswith("*"):
                return float(line.split(":", 1)[1].strip().split("Mhz")[0].split("MHz")[0])
    return None


def measure_sclk(fn, launches=300):
    """The shader clock (and board power) while `fn` runs back to back
    (`launches` calls, outside the timed steps): sysfs samples taken until
    the work drains, the first fifth (ramp-up) dropped."""
    import torch
    sclk_path, power_path = _clock_files()
    if sclk_path is None:
        return None
    fn()
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    for _ in range(launches):
        fn()
    done.record()
    clk, pwr = [], []
    while not done.query():
        try:
            v = _read_sclk_mhz(sclk_path)
            if v is not None:
                clk.append(v)
            if power_path:
                with open(power_path) as f:
                    pwr.append(int(f.read().strip()) / 1e6)
        except (OSError, ValueError, IndexError):
            return None
        time.sleep(0.002)
    torch.cuda.synchronize()
    if not clk:
        return None
    c = np.array(clk[len(clk) // 5:] or clk)
    out = {"mean_mhz": float(c.mean()), "min_mhz": float(c.min()), "max_mhz": float(c.max()), "samples": len(c),
           "source": f"{sclk_path} (current level) during {launches} back-to-back calls of the timed GEMM"}
    if pwr:
        w = np.array(pwr[len(pwr) // 5:] or pwr)
        out["board_power_w"] = float(w.mean())
    return out


def library_ceiling():
    """Time the vendor library (hipBLASLt through torch) on the dense Fprop
    shape with random data: plain f16 and bf16 GEMMs and the per-tensor-scaled
    FP8 GEMM.  None of them does block scaling or per-128 promotion; they are
    the practical ceilings of the matrix cores on this shape and data."""
    import torch
    dev = torch.device("cuda:0")

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    g = torch.Generator(device=dev).manual_seed(0)
    for name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        a = torch.randn(M, K, device=dev, generator=g).to(dt)
        b = torch.randn(N, K, device=dev, generator=g).to(dt)
        ms = timed(lambda: a @ b.t())
        out[f"matmul_{name}"] = {"ms": ms, "TFLOP/s": 2.0 * M * N * K / ms / 1e9}
        del a, b
    a = torch.randn(M, K, device=dev, generator=g).to(torch.float8_e4m3fn)
    b = torch.randn(N, K, device=dev, generator=g).to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    ms = timed(lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
    out["scaled_mm_fp8_per_tensor"] = {"ms": ms, "TFLOP/s": 2.0 * M * N * K / ms / 1e9}
    print(json.dumps({"library_ceiling": out, "shape": [M, N, K], "data": "torch.randn"}), flush=True)


def settle(step_fns, seconds):
    """Run the step back to back for `seconds` before the warmup steps (not
    timed, not counted as warmup): after the GPU has idled (input generation,
    host work) its shader clock ramps up over the first ~30-80 ms of
    sustained load, and a 20-step timed region would otherwise measure the
    ramp rather than the kernels.  Returns the number of steps run."""
    import torch
    if seconds <= 0:
        return 0
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for fn in step_fns:
            fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_steps(step_fns, steps, warmup):
    """Run the kernels of a step `warmup` times, then `steps` times with a HIP
    event around each (events on torch's current stream, which the binding
    passes to the library).  Returns (ms per step from the host clock,
    [mean ms per kernel])."""
    import torch
    for _ in range(warmup):
        for fn in step_fns:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(step_fns) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        for j, fn in enumerate(step_fns):
            fn()
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(len(step_fns))]
    return wall, per


# ---- the other workloads -----------------------------------------------------------------
#
# Each builder returns (kernels, flops, config); a kernel is
# (name, fn, work, unit[, hbm_bytes]) with work in bytes ("GB/s") or in
# GFLOP x 1e3 ("TFLOP/s"); a GEMM whose floor is the memory (the grouped
# ones) also gives its algorithmic HBM bytes.

def _to_bf16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def build_expert_backward(d, accum, dev):
    import torch
    import block_scaled_gemm_amd as bs
    dY, X, W = _to_bf16(d["dY"], dev), _to_bf16(d["X"], dev), _to_bf16(d["W"], dev)
    T, Nw, Kw = 8192, 2048, 7168
    # forward-pass products the backward pass starts from
    qx, sx = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32)
    _, sw, qwt = bs.fp8_quant_block(W, bs.SCALE_FP32, transpose=True)
    del X, W
    out = {}
    dx = torch.empty((T, Kw), dtype=torch.float32, device=dev)
    dw = torch.empty((Nw, Kw), dtype=torch.float32, device=dev)
    qxt = torch.empty((Kw, T), dtype=torch.uint8, device=dev)
    sxt = torch.empty((T // 128, Kw), dtype=torch.float32, device=dev)

    def dual():
        out["qr"], out["sr"], out["qc"], out["sc"] = bs.fp8_quant_dual(dY, bs.SCALE_FP32)
    kernels = [
        ("quant_dual dY[8192x2048]", dual, T * Nw * 4 + 2 * (T * Nw // 128) * 4, "GB/s"),
        ("requant_col X[8192x7168]", lambda: bs.fp8_requant_col(qx, sx, bs.SCALE_FP32, qt=qxt, st=sxt),
         T * Kw * 2 + 2 * (T * Kw // 128) * 4, "GB/s"),
        ("dgrad 8192x7168x2048", lambda: bs.fp8_gemm_blockscaled(
            out["qr"], out["sr"], qwt, sw, bs.BSCALE_BLOCK, 1, sw.stride(0), bs.OUT_F32, d=dx, accum=accum),
         2.0 * T * Kw * Nw / 1e3, "TFLOP/s"),
        ("wgrad 2048x7168x8192", lambda: bs.fp8_gemm_blockscaled(
            out["qc"], out["sc"], qxt, sxt, bs.BSCALE_TILE, sxt.stride(0), 0, bs.OUT_F32, d=dw, accum=accum),
         2.0 * Nw * Kw * T / 1e3, "TFLOP/s"),
    ]
    config = {"workload": "expert backward: quant dY[8192x2048] 1x128 and 128x1 in one pass + re-tile "
                          "X[8192x7168] 1x128 -> 128x1 + Dgrad 8192x7168x2048 + Wgrad 2048x7168x8192 -> fp32"}
    return kernels, 4.0 * T * Kw * Nw, config


def build_grouped(name, d, accum, dev):
    import torch
    import block_scaled_gemm_amd as bs
    G, Ng, Kg = d["W"].shape
    offsets = torch.from_numpy(d["offsets"]).to(dev)
    rows = int(d["offsets"][-1])
    Xc, Wc = _to_bf16(d["Xcat"], dev), _to_bf16(d["W"].reshape(G * Ng, Kg), dev)
    mode = bs.SCALE_POW2 if name == "grouped_upproj" else bs.SCALE_FP32
    qx = torch.empty((rows, Kg), dtype=torch.uint8, device=dev)
    sx = torch.empty((Kg // 128, rows), dtype=torch.float32, device=dev)
    qw = torch.empty((G * Ng, Kg), dtype=torch.uint8, device=dev)
    sw = torch.empty((G * Ng // 128, Kg // 128), dtype=torch.float32, device=dev)
    y = torch.empty((rows, Ng), dtype=torch.bfloat16, device=dev)
    # algorithmic HBM bytes of the grouped GEMM: every weight code and block
    # scale once, the activations' codes and scales, the bf16 output
    gemm_bytes = G * Ng * Kg + G * (Ng // 128) * (Kg // 128) * 4 + rows * Kg + rows * (Kg // 128) * 4 + rows * Ng * 2
    kernels = [
        (f"quant_tile X[{rows}x{Kg}]", lambda: bs.fp8_quant_tile(Xc, bs.AXIS_ROW, mode, q=qx, s=sx),
         quant_bytes_row(rows, Kg), "GB/s"),
        (f"quant_block W[{G}x{Ng}x{Kg}]", lambda: bs.fp8_quant_block(Wc, mode, q=qw, s=sw),
         quant_bytes_block(G * Ng, Kg), "GB/s"),
        (f"grouped GEMM G={G} rows={rows} N={Ng} K={Kg}", lambda: bs.fp8_grouped_gemm(
            offsets, qx, sx, qw.view(G, Ng, Kg), sw.view(G, Ng // 128, Kg // 128), bs.OUT_BF16, d=y, accum=accum),
         2.0 * rows * Ng * Kg / 1e3, "TFLOP/s", gemm_bytes),
    ]
    config = {"workload": f"{name}: quant X[{rows}x{Kg}] 1x128 + quant W[{G}x{Ng}x{Kg}] 128x128 + grouped "
                          f"GEMM ({G} experts, {rows} rows, N={Ng}, K={Kg}) -> bf16",
              "scales": "pow2" if mode == bs.SCALE_POW2 else "fp32"}
    return kernels, 2.0 * rows * Ng * Kg, config


def build_moe_backward(d, accum, dev):
    import torch
    import block_scaled_gemm_amd as bs
    from block_scaled_gemm_amd import inputs
    G, Nw, Kw = d["W"].shape
    offs_h = d["offsets"]
    rows = int(offs_h[-1])
    offsets = torch.from_numpy(offs_h).to(dev)
    dY = _to_bf16(inputs.random_bf16(213, (rows, Nw), sd=1e-3), dev)
    X = _to_bf16(d["Xcat"], dev)
    _, sw, qwt = bs.fp8_quant_block(_to_bf16(d["W"].reshape(G * Nw, Kw), dev), bs.SCALE_FP32, transpose=True)
    kb = bs.grouped_col_bound(rows, G)
    qd = torch.empty((rows, Nw), dtype=torch.uint8, device=dev)
    sd = torch.empty((Nw // 128, rows), dtype=torch.float32, device=dev)
    dx = torch.empty((rows, Kw), dtype=torch.float32, device=dev)
    qdt = torch.zeros((Nw, kb), dtype=torch.uint8, device=dev)
    sdt = torch.ones((kb // 128, Nw), dtype=torch.float32, device=dev)
    qxt = torch.zeros((Kw, kb), dtype=torch.uint8, device=dev)
    sxt = torch.ones((kb // 128, Kw), dtype=torch.float32, device=dev)
    dw = torch.empty((G, Nw, Kw), dtype=torch.float32, device=dev)
    L = bs.lib()
    st = lambda: torch.cuda.current_stream().cuda_stream

    def gcol(x, q, s_):
        bs._check(L.fp8_quant_tile_grouped_col(x.data_ptr(), rows, x.shape[1], x.stride(0), G, offsets.data_ptr(),
                                               bs.SCALE_FP32, q.data_ptr(), q.stride(0), s_.data_ptr(),
                                               s_.stride(0), st()), "fp8_quant_tile_grouped_col")
    colb = lambda c: rows * c * 3 + 2 * 4 * (kb // 128) * c  # bf16 in, codes out, scales
    kernels = [
        (f"quant_tile dY[{rows}x{Nw}]", lambda: bs.fp8_quant_tile(dY, bs.AXIS_ROW, bs.SCALE_FP32, q=qd, s=sd),
         quant_bytes_row(rows, Nw), "GB/s"),
        (f"moe dgrad G={G} rows={rows} {Kw}x{Nw}", lambda: bs.fp8_grouped_gemm_strided(
            offsets, qd, sd, G, Kw, qwt, qwt.stride(0), Nw, sw, bs.BSCALE_BLOCK, 1, sw.stride(0),
            (Nw // 128) * sw.stride(0), bs.OUT_F32, d=dx, accum=accum), 2.0 * rows * Kw * Nw / 1e3, "TFLOP/s",
         G * Nw * Kw + rows * Nw + rows * Kw * 4),
        (f"quant_grouped_col dY[{rows}x{Nw}]", lambda: gcol(dY, qdt, sdt), colb(Nw), "GB/s"),
        (f"quant_grouped_col X[{rows}x{Kw}]", lambda: gcol(X, qxt, sxt), colb(Kw), "GB/s"),
        (f"moe wgrad K-grouped G={G} {Nw}x{Kw}", lambda: bs.fp8_grouped_gemm_kgrouped(
            offsets, qdt, sdt, qxt, sxt, bs.OUT_F32, d=dw, accum=accum), 2.0 * rows * Nw * Kw / 1e3, "TFLOP/s",
         (Nw + Kw) * kb + G * Nw * Kw * 4),
    ]
    config = {"workload": f"moe_backward: {G} up-projection experts, {rows} routed rows, W_e[{Nw}x{Kw}]: "
                          f"quant dY 1x128 + M-grouped Dgrad + dY and X 128x1 per expert + K-grouped Wgrad -> fp32"}
    return kernels, 4.0 * rows * Nw * Kw, config


PEAK_UNIT = {"TFLOP/s": (PEAK_FP8_TFLOPS, "mfma"), "GB/s": (PEAK_HBM_GBPS, "hbm")}


def run_kernels(kernels, flops, config, steps, warmup, settle_s=0.0):
    """Time a workload's step; returns its report (the line's fields)."""
    n_settle = settle([k[1] for k in kernels], settle_s)
    wall, per = time_steps([k[1] for k in kernels], steps, warmup)
    report = {}
    for k, ms in zip(kernels, per):
        kname, _, work, unit = k[:4]
        ach = work / (ms * 1e-3) / 1e9  # GB/s for bytes, TFLOP/s for flops / 1e3
        peak, _ = PEAK_UNIT[unit]
        row = {"ms": ms, unit: ach, "frac": ach / peak}
        if len(k) > 4:  # a GEMM bound by memory: its bytes against HBM too
            gbs = k[4] / (ms * 1e-3) / 1e9
            row.update({"GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBPS})
        report[kname] = row
    dom = int(np.argmax(per))
    kname, _, work, unit = kernels[dom][:4]
    if len(kernels[dom]) > 4:
        ach, peak, unit2, bound = report[kname]["GB/s"], PEAK_HBM_GBPS, "GB/s", "hbm"
    else:
        peak, bound = PEAK_UNIT[unit]
        ach, unit2 = report[kname][unit], unit
    return {"value": flops / (wall * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": wall, "config": config,
            "settle": {"seconds": settle_s, "steps": n_settle},
            "roofline": {"bound": bound, "achieved": ach, "peak": peak, "unit": unit2, "frac": ach / peak,
                         "traffic": measured_traffic(kname), "kernel": kname, "kernel_ms": per[dom]},
            "kernels": report}


def build_dense(d, dev):
    """The dense Fprop's kernels for --profile-kernels: the default line's
    quantisers and GEMM, plus the GEMM in the exact mode and in the
    power-of-two mode (on power-of-two quantisations)."""
    import torch
    import block_scaled_gemm_amd as bs
    X, W = _to_bf16(d["X"], dev), _to_bf16(d["W"], dev)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32, q=qx, s=sx)
    bs.fp8_quant_block(W, bs.SCALE_FP32, q=qw, s=sw)
    qx2, sx2 = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_POW2)
    qw2, sw2, _ = bs.fp8_quant_block(W, bs.SCALE_POW2)
    # algorithmic bytes: both operands' codes and scales once, the bf16 output once
    ideal = M * K + N * K + (K // 128) * M * 4 + (N // 128) * (K // 128) * 4 + M * N * 2
    gemm = lambda a, sa, b, sb, acc: (lambda: bs.fp8_gemm_blockscaled(a, sa, b, sb, bs.BSCALE_BLOCK, K // 128, 1,
                                                                      bs.OUT_BF16, d=y, accum=acc))
    F = 2.0 * M * N * K / 1e3
    return [
        (f"quant_tile X[{M}x{K}]", lambda: bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32, q=qx, s=sx),
         quant_bytes_row(M, K), "GB/s"),
        (f"quant_block W[{N}x{K}]", lambda: bs.fp8_quant_block(W, bs.SCALE_FP32, q=qw, s=sw),
         quant_bytes_block(N, K), "GB/s"),
        (DENSE_GEMM_LABEL, gemm(qx, sx, qw, sw, bs.ACCUM_MFMA8), F, "TFLOP/s", ideal),
        (f"gemm {M}x{N}x{K} (exact group partials, f16 matrix cores)", gemm(qx, sx, qw, sw, bs.ACCUM_FP32), F,
         "TFLOP/s", ideal),
        (f"gemm {M}x{N}x{K} (power-of-two scales inside the FP8 MFMA)", gemm(qx2, sx2, qw2, sw2,
                                                                            bs.ACCUM_MFMA8_POW2), F, "TFLOP/s",
         ideal),
    ]


def profile_kernels():
    """Every workload kernel on its own: a marker dispatch (torch's spin
    kernel), PROFILE_CALLS launches of the kernel, a second marker, then a
    synchronisation -- the layout --summarize-profile splits rocprofv3's
    per-dispatch records by (whatever runs between a closing marker and the
    next opening one, such as building the next workload's inputs, is not
    counted).  Prints the manifest (labels in launch order, algorithmic
    work) as one JSON line."""
    import torch
    from block_scaled_gemm_amd import inputs
    import block_scaled_gemm_amd as bs
    if not hasattr(torch.cuda, "_sleep"):
        raise RuntimeError("torch.cuda._sleep (the marker dispatch) is missing")
    dev = torch.device("cuda:0")
    manifest = []

    def run(workload, kernels):
        for k in kernels:  # warm, before any marker
            k[1]()
        torch.cuda.synchronize()
        for k in kernels:
            torch.cuda._sleep(1000)  # opens the kernel's segment
            for _ in range(PROFILE_CALLS):
                k[1]()
            torch.cuda._sleep(1000)  # closes it
            torch.cuda.synchronize()
            manifest.append({"workload": workload, "label": k[0], "calls": PROFILE_CALLS, "work": k[2],
                             "unit": k[3], "bytes": k[4] if len(k) > 4 else (k[2] if k[3] == "GB/s" else None)})
        log(f"profiled {workload} ({len(kernels)} kernels)")

    run("dense_fprop", build_dense(inputs.dense_fprop(), dev))
    torch.cuda.empty_cache()
    run("expert_backward", build_expert_backward(inputs.expert_backward(), bs.ACCUM_MFMA8, dev)[0])
    torch.cuda.empty_cache()
    up = inputs.grouped_upproj()
    run("grouped_upproj", build_grouped("grouped_upproj", up, bs.ACCUM_MFMA8_POW2, dev)[0])
    torch.cuda.empty_cache()
    run("moe_backward", build_moe_backward(up, bs.ACCUM_MFMA8, dev)[0])
    del up
    torch.cuda.empty_cache()
    run("decode_grouped", build_grouped("decode_grouped", inputs.decode_grouped(), bs.ACCUM_MFMA8, dev)[0])
    print(json.dumps({"profile_manifest": manifest, "source_hash": source_hash(PROFILE_SOURCES)}), flush=True)


MARKER = "spin_kernel"  # torch.cuda._sleep's kernel
_PK = "python3 /root/repo/bench.py --profile-kernels"
PROFILE_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    f"rocprofv3 --kernel-trace --output-format csv -d <out>/trace -o p -- {_PK} > <out>/manifest.json",
    f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o p -- {_PK}",
    f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o p -- {_PK}",
    "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU GRBM_GUI_ACTIVE --output-format csv "
    f"-d <out>/sq -o p -- {_PK}",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/probe_fetch -o p -- "
    "python3 /root/repo/bench.py --traffic-probe",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/probe_write -o p -- "
    "python3 /root/repo/bench.py --traffic-probe",
    "python3 /root/repo/bench.py --summarize-profile <out> <out>/manifest.json",
]


def _csv_rows(root, suffix):
    import csv
    rows = []
    for dirpath, _, names in sorted(os.walk(root)):
        for n in sorted(names):
            if n.endswith(suffix):
                with open(os.path.join(dirpath, n), newline="") as f:
                    rows.extend(csv.DictReader(f))
    return rows


def _short(name):
    import re
    n = re.sub(r"^void ", "", name)
    n = n.replace("fp8bs::", "")
    return re.sub(r"\(.*$", "", n).strip()


def _dispatches(root, suffix):
    """[(dispatch id, kernel name, {counter: value} or duration ns)] in
    dispatch order from one rocprofv3 pass."""
    rows = _csv_rows(root, suffix)
    if not rows:
        raise RuntimeError(f"no *{suffix} under {root}")
    key = "Dispatch_Id" if "Dispatch_Id" in rows[0] else "Correlation_Id"
    by = {}
    for r in rows:
        i = int(r[key])
        name = r["Kernel_Name"]
        if "Counter_Name" in r:
            e = by.setdefault(i, (name, {}))
            e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        else:
            by[i] = (name, int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [(i, by[i][0], by[i][1]) for i in sorted(by)]


def _segments(disp, n):
    """The dispatches between the opening and the closing marker of each of
    the n kernels (markers come in pairs)."""
    marks = [k for k, (_, name, _) in enumerate(disp) if MARKER in name]
    if len(marks) != 2 * n:
        names = sorted({_short(x[1]) for x in disp})[:20]
        raise RuntimeError(f"{len(marks)} marker dispatches for {n} kernels (two each); kernels seen: {names}")
    return [disp[marks[2 * k] + 1:marks[2 * k + 1]] for k in range(n)]


def _probe_factor(root, counter, true_bytes):
    """Counter bytes per true byte for the copy probe (the largest dispatch
    of the probe run)."""
    disp = _dispatches(root, "counter_collection.csv")
    kib = max(v.get(counter, 0.0) for _, _, v in disp)
    return kib * 1024.0 / true_bytes


def summarize_profile(root, manifest_path, out_path, command):
    """The per-kernel summary from the rocprofv3 passes under `root`
    (subfolders trace/, fetch/, write/, sq/, probe_fetch/, probe_write/) and
    the manifest line that --profile-kernels printed; written as text with
    the machine-readable `traffic | label | bytes` lines."""
    with open(manifest_path) as f:
        man = next(json.loads(ln) for ln in f if ln.startswith("{") and "profile_manifest" in ln)
    entries = man["profile_manifest"]
    n = len(entries)
    seg = {}
    seg["trace"] = _segments(_dispatches(os.path.join(root, "trace"), "kernel_trace.csv"), n)
    for p in ("fetch", "write", "sq"):
        seg[p] = _segments(_dispatches(os.path.join(root, p), "counter_collection.csv"), n)
    probe = 1 << 30  # torch.neg over 2^28 fp32: 1 GiB read, 1 GiB written
    ff = _probe_factor(os.path.join(root, "probe_fetch"), "FETCH_SIZE", probe)
    wf = _probe_factor(os.path.join(root, "probe_write"), "WRITE_SIZE", probe)
    lines = [
        "# Per-launch time, HBM traffic and matrix-core / VALU activity of every workload kernel (one MI355X)",
        "",
        "Commands (each kernel launched on its own after a marker dispatch; one rocprofv3 pass per row):",
        "",
    ]
    lines += ["    " + c for c in command]
    lines += [
        "",
        f"Counter scaling from the copy probe (torch.neg, 1 GiB read + 1 GiB written): FETCH_SIZE {ff:.4f} "
        f"counter bytes per byte read, WRITE_SIZE {wf:.4f} per byte written; traffic = FETCH/{ff:.4f} + "
        f"WRITE/{wf:.4f}.  Clock = (GRBM_GUI_ACTIVE / 8 XCDs) / duration; MFMA busy = "
        "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); VALU = 4 x SQ_INSTS_VALU / (1024 x cycles).  "
        "Short kernels (< 50 us) get an overstated clock window, so their busy fractions are left out.",
        "",
        "| workload | kernel (label) | HIP kernels | us/launch | MB read | MB written | traffic / algorithmic | "
        "achieved | MFMA busy | VALU | clock GHz |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    machine = []
    for k, e in enumerate(entries):
        calls = e["calls"]
        names = sorted({_short(x[1]) for x in seg["trace"][k]})
        us = sum(x[2] for x in seg["trace"][k]) / calls / 1e3
        rd = sum(x[2].get("FETCH_SIZE", 0.0) for x in seg["fetch"][k]) * 1024.0 / ff / calls
        wr = sum(x[2].get("WRITE_SIZE", 0.0) for x in seg["write"][k]) * 1024.0 / wf / calls
        sq = {}
        for x in seg["sq"][k]:
            for c, v in x[2].items():
                sq[c] = sq.get(c, 0.0) + v / calls
        alg = e.get("bytes")
        ratio = f"{(rd + wr) / alg:.2f}" if alg else "-"
        if e["unit"] == "GB/s":
            ach = f"{e['work'] / (us * 1e-6) / 1e9:.0f} GB/s"
        else:
            ach = f"{e['work'] * 1e3 / (us * 1e-6) / 1e12:.0f} TFLOP/s"
        cyc = sq.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        if us >= 50 and cyc > 0:
            ghz = cyc / (us * 1e3)
            mfma = f"{100 * sq.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / (1024 * cyc):.1f}%"
            valu = f"{100 * 4 * sq.get('SQ_INSTS_VALU', 0.0) / (1024 * cyc):.1f}%"
            clk = f"{ghz:.2f}"
        else:
            mfma = valu = clk = "-"
        lines.append(f"| {e['workload']} | {e['label']} | {', '.join(f'`{x}`' for x in names)} | {us:.1f} | "
                     f"{rd / 1e6:.1f} | {wr / 1e6:.1f} | {ratio} | {ach} | {mfma} | {valu} | {clk} |")
        machine.append(f"traffic | {e['label']} | {rd + wr:.0f}")
    lines += ["", "Machine-readable (bench.py reads these while the kernel sources are unchanged):", "",
              f"source_hash: {man['source_hash']}"] + machine
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def other_workload(name, args, data=None):
    """One of the other workloads (see the module docstring); returns its
    report."""
    import torch
    import block_scaled_gemm_amd as bs
    from block_scaled_gemm_amd import inputs
    dev = torch.device("cuda:0")
    accum_name = args.accum
    if accum_name is None:
        accum_name = "mfma8_pow2" if name == "grouped_upproj" else "mfma8"
    accum = {"fp32": bs.ACCUM_FP32, "mfma8": bs.ACCUM_MFMA8, "mfma8_pow2": bs.ACCUM_MFMA8_POW2}[accum_name]
    if name == "expert_backward":
        built = build_expert_backward(data or inputs.expert_backward(), accum, dev)
    elif name == "moe_backward":
        built = build_moe_backward(data or inputs.grouped_upproj(), accum, dev)
    else:
        d = data or (inputs.grouped_upproj() if name == "grouped_upproj" else inputs.decode_grouped())
        built = build_grouped(name, d, accum, dev)
    kernels, flops, config = built
    config["accum"] = accum_name
    rep = run_kernels(kernels, flops, config, args.steps, args.warmup, args.settle)
    del kernels, built
    torch.cuda.empty_cache()
    return rep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity check")
    ap.add_argument("--no-workloads", action="store_true", help="time the dense Fprop only")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of back-to-back steps before the warmup steps, untimed (clock ramp-up)")
    ap.add_argument("--accum", choices=["mfma8", "fp32", "mfma8_pow2"], default=None,
                    help="GEMM accumulation: FP8 matrix cores (mfma8), exact group partials (fp32), or "
                         "power-of-two scales inside the FP8 MFMA (mfma8_pow2; power-of-two scales only); "
                         "default: mfma8_pow2 for grouped_upproj, mfma8 elsewhere")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only a plain copy of known size (counter scaling)")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="launch every workload kernel on its own after a marker dispatch (for rocprofv3 passes)")
    ap.add_argument("--summarize-profile", nargs=2, metavar=("DIR", "MANIFEST"),
                    help="write the per-kernel summary from rocprofv3 passes over --profile-kernels")
    ap.add_argument("--library-ceiling", action="store_true",
                    help="time the vendor GEMMs on the dense shape (context only)")
    ap.add_argument("--workload", default="dense_fprop",
                    choices=["dense_fprop", "expert_backward", "grouped_upproj", "decode_grouped", "moe_backward"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fine-grained FP8 linear here is a "
              "single-GPU build (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.workload == "dense_fprop" and args.accum == "mfma8_pow2":
        print("bench.py: the dense Fprop quantises with FP32 scales; it reports the power-of-two mode "
              "under gemm_modes", file=sys.stderr)
        sys.exit(2)
    if args.accum == "mfma8_pow2" and args.workload not in ("grouped_upproj",):
        print("bench.py: mfma8_pow2 needs power-of-two scales; only grouped_upproj quantises with them",
              file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe()
        return
    if args.profile_kernels:
        profile_kernels()
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile[0], args.summarize_profile[1], PROFILE_SUMMARY,
                          PROFILE_COMMANDS)
        return
    if args.library_ceiling:
        library_ceiling()
        return
    if args.workload != "dense_fprop":
        rep = other_workload(args.workload, args)
        line = {"metric": METRIC, "value": rep["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": rep["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
                "data": "synthetic (seeded numpy, shapes and distributions of the workload)",
                "config": rep["config"], "settle": rep["settle"], "roofline": rep["roofline"],
                "kernels": rep["kernels"], "cpu_baseline": None}
        print(json.dumps(line), flush=True)
        return

    import torch
    import block_scaled_gemm_amd as bs
    from block_scaled_gemm_amd import inputs
    accum_name = args.accum or "mfma8"
    accum = {"fp32": bs.ACCUM_FP32, "mfma8": bs.ACCUM_MFMA8}[accum_name]
    other = "mfma8" if accum_name == "fp32" else "fp32"
    kernel = GEMM_KERNEL[accum_name]

    t_gen = time.perf_counter()
    d = inputs.dense_fprop()
    Xh, Wh = d["X"], d["W"]
    dev = torch.device("cuda:0")
    X = _to_bf16(Xh, dev)
    W = _to_bf16(Wh, dev)
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f} s")

    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32, q=qx, s=sx)
        if ev is not None:
            ev[1].record()
        bs.fp8_quant_block(W, bs.SCALE_FP32, q=qw, s=sw)
        if ev is not None:
            ev[2].record()
        bs.fp8_gemm_blockscaled(qx, sx, qw, sw, bs.BSCALE_BLOCK, K // 128, 1, bs.OUT_BF16, d=y, accum=accum)
        if ev is not None:
            ev[3].record()

    n_settle = settle([step], args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"settle ({n_settle} steps, {args.settle} s) and warmup done ({args.warmup} steps)")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qx_ms = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    qw_ms = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    gemm_ms = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = wall * 1e3 / args.steps
    log(f"{args.steps} steps: {step_ms:.3f} ms/step (quant X {qx_ms:.3f}, quant W {qw_ms:.3f}, gemm {gemm_ms:.3f} ms)")
    # the timed step's results, for the parity check against the oracle
    timed_out = None
    if not args.no_cpu:
        timed_out = {"y": y.view(torch.int16).cpu().numpy().view(np.uint16), "qx": qx.cpu().numpy(),
                     "sx": sx.cpu().numpy(), "qw": qw.cpu().numpy(), "sw": sw.cpu().numpy()}

    # outside the timed steps: the same GEMM in the other accumulation mode,
    # and the power-of-two-scale mode on power-of-two quantisations of X, W
    def gemm_time(fn):
        fn()
        oe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in oe:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in oe]))

    gemm_fn = lambda: bs.fp8_gemm_blockscaled(qx, sx, qw, sw, bs.BSCALE_BLOCK, K // 128, 1, bs.OUT_BF16, d=y,
                                              accum=accum)
    sclk = measure_sclk(gemm_fn)
    other_accum = bs.ACCUM_MFMA8 if accum == bs.ACCUM_FP32 else bs.ACCUM_FP32
    other_ms = gemm_time(lambda: bs.fp8_gemm_blockscaled(qx, sx, qw, sw, bs.BSCALE_BLOCK, K // 128, 1, bs.OUT_BF16,
                                                         d=y, accum=other_accum))
    qx2, sx2 = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_POW2)
    qw2, sw2, _ = bs.fp8_quant_block(W, bs.SCALE_POW2)
    pow2_ms = gemm_time(lambda: bs.fp8_gemm_blockscaled(qx2, sx2, qw2, sw2, bs.BSCALE_BLOCK, K // 128, 1,
                                                        bs.OUT_BF16, d=y, accum=bs.ACCUM_MFMA8_POW2))
    del qx2, sx2, qw2, sw2, X, W, qx, sx, qw, sw, y
    torch.cuda.empty_cache()

    flops = 2.0 * M * N * K
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    bx, bw = quant_bytes_row(M, K), quant_bytes_block(N, K)
    traffic = measured_traffic(DENSE_GEMM_LABEL if accum_name == "mfma8" else
                               f"gemm {M}x{N}x{K} (exact group partials, f16 matrix cores)")
    flops_tf = lambda ms: flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded numpy: N(0,1) with 0.1% x100 outliers; N(0,0.02))",
        "config": {"workload": "dense Fprop: quant X[4096x7168] 1x128 + quant W[18432x7168] 128x128 "
                               "+ GEMM 4096x18432x7168 -> bf16",
                   "M": M, "N": N, "K": K, "scales": "fp32", "accum": accum_name},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tflops / PEAK_FP8_TFLOPS,
                     "traffic": traffic, "kernel": kernel, "kernel_ms": gemm_ms},
        "settle": {"seconds": args.settle, "steps": n_settle},
        "parity": None,
        "sclk": sclk,
        "gemm_modes": {
            accum_name: {"ms": gemm_ms, "TFLOP/s": flops_tf(gemm_ms),
                         "frac_fp8_peak": flops_tf(gemm_ms) / PEAK_FP8_TFLOPS},
            other: {"ms": other_ms, "TFLOP/s": flops_tf(other_ms),
                    "frac_fp8_peak": flops_tf(other_ms) / PEAK_FP8_TFLOPS},
            "mfma8_pow2 (power-of-two scales)": {"ms": pow2_ms, "TFLOP/s": flops_tf(pow2_ms),
                                                 "frac_fp8_peak": flops_tf(pow2_ms) / PEAK_FP8_TFLOPS},
        },
        "quantizers": {
            "quant_tile_row_X": {"ms": qx_ms, "GB/s": bx / (qx_ms * 1e-3) / 1e9,
                                 "frac_hbm": bx / (qx_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
            "quant_block_W": {"ms": qw_ms, "GB/s": bw / (qw_ms * 1e-3) / 1e9,
                              "frac_hbm": bw / (qw_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        },
        "workloads": None,
        "cpu_baseline": None,
    }

    if not args.no_workloads:
        wl = {}
        t_w = time.perf_counter()
        wl["expert_backward"] = other_workload("expert_backward", argparse.Namespace(
            accum=None, steps=args.steps, warmup=args.warmup, settle=args.settle))
        log(f"expert_backward timed ({time.perf_counter() - t_w:.1f} s)")
        up = inputs.grouped_upproj()
        for name in ("grouped_upproj", "moe_backward"):
            wl[name] = other_workload(name, argparse.Namespace(accum=None, steps=args.steps, warmup=args.warmup,
                                                               settle=args.settle), data=up)
            log(f"{name} timed ({time.perf_counter() - t_w:.1f} s)")
        del up
        wl["decode_grouped"] = other_workload("decode_grouped", argparse.Namespace(
            accum=None, steps=args.steps, warmup=args.warmup, settle=args.settle))
        log(f"decode_grouped timed ({time.perf_counter() - t_w:.1f} s)")
        out["workloads"] = wl

    if not args.no_cpu:
        log("timing the CPU oracle on a sub-block")
        base, sample = cpu_baseline(Xh, Wh)
        log("timing the CPU quantisers")
        base["quantizers"] = cpu_quant_baseline(Xh, Wh)
        out["cpu_baseline"] = base
        log("parity of the timed output against the oracle on the same sample")
        out["parity"] = parity(sample, timed_out["y"], timed_out["qx"], timed_out["sx"], timed_out["qw"],
                               timed_out["sw"], accum)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

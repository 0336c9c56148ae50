"""GPU block-scaled GEMM against the CPU oracle.

The inputs are quantised on the GPU (codes and scales checked bit-exact
against the oracle's), then the GPU GEMM is compared with the oracle's
exact-group-partial FP64 result through the comparator of oracle/compare.py
(gpu_util.check): every mode must have max|D - R| / max|R| <= 1e-3 (fp32
output) or 8e-3 (bf16); the exact mode must also meet the same tolerance
elementwise (each |D - R| over max(|R|, 1% of max|R|)); the FP8-matrix-core
modes must stay within their per-element bound 2^-10 * R_abs + output
rounding, their elementwise figure being logged.  The workloads at their
real sizes are compared on every output."""
import functools

import numpy as np
import pytest
import torch

import oracle
from block_scaled_gemm_amd import inputs
from gpu_util import workload, bf16_f64, check, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu

ACCUMS = pytest.mark.parametrize("accum", [0, 1], ids=["acc32", "mfma8"])
# the power-of-two scaled-MFMA mode joins wherever every scale is a power of two
ACCUMS_POW2 = pytest.mark.parametrize("accum", [0, 1, 2], ids=["acc32", "mfma8", "mfma8pow2"])


def out_f64(t):
    h = host(t)
    return bf16_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


def quant_both(hip, orc, x, kind, mode):
    """Quantise on the GPU and on the CPU, require bit-exact equality and
    return the GPU tensors and the host copies."""
    if kind == "row":
        q, s = hip.fp8_quant_tile(dev_bf16(x), hip.AXIS_ROW, mode)
        wq, ws = orc.quant_tile(x, 0, mode)
        qt = wqt = None
    elif kind == "col":
        q, s = hip.fp8_quant_tile(dev_bf16(x), hip.AXIS_COL, mode)
        wq, ws = orc.quant_tile(x, 1, mode)
        qt = wqt = None
    else:
        q, s, qt = hip.fp8_quant_block(dev_bf16(x), mode, transpose=True)
        wq, ws, wqt = orc.quant_block(x, mode, transpose=True)
        np.testing.assert_array_equal(host(qt), wqt)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))
    return q, s, qt, wq, ws, wqt


def full(orc, a, sa, b, sb, kind, s0, s1):
    """Oracle result and its absolute-value companion R_abs."""
    return orc.gemm(a, sa, b, sb, kind, s0, s1), orc.gemm_abs(a, sa, b, sb, kind, s0, s1)




@ACCUMS
@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
def test_tiny_fprop(hip, orc, out, accum):
    """Workload 0 in full: X[128x512] 1x128 tiles, W[256x512] 128x128 blocks."""
    d = workload("tiny_fprop")
    qx, sx, _, wqx, wsx, _ = quant_both(hip, orc, d["X"], "row", 0)
    qw, sw, _, wqw, wsw, _ = quant_both(hip, orc, d["W"], "block", 0)
    y = hip.linear_fprop(qx, sx, qw, sw, out, accum=accum)
    r, rabs = full(orc, wqx, wsx, wqw, wsw, 0, wsw.shape[1], 1)
    check(out_f64(y), r, rabs, out, accum, 4, f"tiny fprop out={out} accum={accum}")


@ACCUMS_POW2
@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_linear_three_gemms_ragged(hip, orc, mode, out, accum):
    """Fprop, Dgrad and Wgrad at sizes spanning several tiles with ragged
    tails: Fprop X[300x1024] W[260x1024]; Dgrad dY[384x256] W[256x1024];
    Wgrad dY^T X2 with 384 tokens, X2[384x200]."""
    if accum == 2 and mode == 0:
        pytest.skip("the scaled-MFMA mode takes power-of-two scales only")
    X = inputs.random_bf16(101, (300, 1024))
    W = inputs.random_bf16(102, (260, 1024), sd=0.02, outliers=False)
    qx, sx, _, wqx, wsx, _ = quant_both(hip, orc, X, "row", mode)
    qw, sw, _, wqw, wsw, _ = quant_both(hip, orc, W, "block", mode)
    y = hip.linear_fprop(qx, sx, qw, sw, out, accum=accum)
    r, rabs = full(orc, wqx, wsx, wqw, wsw, 0, wsw.shape[1], 1)
    check(out_f64(y), r, rabs, out, accum, 8, f"ragged fprop mode={mode} out={out} accum={accum}")
    # Dgrad: the contraction runs over W's 256 rows (a multiple of 128)
    Wd = W[:256]
    dY = inputs.random_bf16(103, (384, 256), sd=1e-3)
    qd, sd_, _, wqd, wsd, _ = quant_both(hip, orc, dY, "row", mode)
    qwd, swd, qwdt, wqwd, wswd, wqwdt = quant_both(hip, orc, Wd, "block", mode)
    dx = hip.linear_dgrad(qd, sd_, qwdt, swd, out, accum=accum)
    r, rabs = full(orc, wqd, wsd, wqwdt, wswd, 0, 1, wswd.shape[1])
    check(out_f64(dx), r, rabs, out, accum, 2, f"ragged dgrad mode={mode} out={out} accum={accum}")
    # Wgrad: A = dY^T (128x1 tiles along tokens), B = X2^T (same)
    X2 = inputs.random_bf16(104, (384, 200))
    qdt, sdt, _, wqdt, wsdt, _ = quant_both(hip, orc, dY, "col", mode)
    qxt, sxt, _, wqxt, wsxt, _ = quant_both(hip, orc, X2, "col", mode)
    dw = hip.linear_wgrad(qdt, sdt, qxt, sxt, out, accum=accum)
    r, rabs = full(orc, wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
    check(out_f64(dw), r, rabs, out, accum, 3, f"ragged wgrad mode={mode} out={out} accum={accum}")


@ACCUMS_POW2
@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
@pytest.mark.parametrize("shape", [(1, 1, 128), (1, 300, 256), (257, 1, 128), (3, 129, 384), (511, 257, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_degenerate_shapes(hip, orc, shape, mode, accum):
    """Fprop at the smallest and most ragged sizes: a single row, a single
    column, a single K group, tiles holding 1-3 rows or columns; bf16 and
    fp32 out into padded outputs (their row stride a multiple of 4)."""
    if accum == 2 and mode == 0:
        pytest.skip("the scaled-MFMA mode takes power-of-two scales only")
    M, N, K = shape
    X = inputs.random_bf16(140 + M, (M, K))
    W = inputs.random_bf16(141 + N, (N, K), sd=0.02, outliers=False)
    qx, sx, _, wqx, wsx, _ = quant_both(hip, orc, X, "row", mode)
    qw, sw, _, wqw, wsw, _ = quant_both(hip, orc, W, "block", mode)
    r, rabs = full(orc, wqx, wsx, wqw, wsw, 0, wsw.shape[1], 1)
    npad = (N + 3) // 4 * 4
    for out in (1, 0):
        dt = torch.float32 if out else torch.bfloat16
        dpad = torch.full((M, npad), 7.0, dtype=dt, device="cuda")
        hip.fp8_gemm_blockscaled(qx, sx, qw, sw, hip.BSCALE_BLOCK, sw.stride(0), 1, out, d=dpad[:, :N], accum=accum)
        check(out_f64(dpad[:, :N]), r, rabs, out, accum, K // 128, f"{M}x{N}x{K} mode={mode} out={out} accum={accum}")
        assert torch.all(dpad[:, N:] == 7.0).item(), "columns past N written"


@pytest.mark.parametrize("accum", [1, 2], ids=["mfma8", "mfma8pow2"])
@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_wide_tiles_ragged(hip, orc, mode, out, accum):
    """The FP8 modes' 256 x 256 tiles with ragged edges (shapes with enough
    tiles that the launch picks them on a 256-CU MI355X): Fprop X[8155x1024]
    W[2008x1024], every tile wide, the last row and column of tiles partial;
    Fprop X[4059x512] W[4196x512], wide tiles up to column 4096 and 256 x 128
    tiles after it; Wgrad over 512 tokens into 8152 x 2008 (per-column
    scales on wide tiles).  Every output compared."""
    if accum == 2 and mode == 0:
        pytest.skip("the scaled-MFMA mode takes power-of-two scales only")
    for i, (m, n, k) in enumerate([(8155, 2008, 1024), (4059, 4196, 512)]):
        X = inputs.random_bf16(131 + 2 * i, (m, k))
        W = inputs.random_bf16(132 + 2 * i, (n, k), sd=0.02, outliers=False)
        qx, sx, _, wqx, wsx, _ = quant_both(hip, orc, X, "row", mode)
        qw, sw, _, wqw, wsw, _ = quant_both(hip, orc, W, "block", mode)
        y = hip.linear_fprop(qx, sx, qw, sw, out, accum=accum)
        r, rabs = full(orc, wqx, wsx, wqw, wsw, 0, wsw.shape[1], 1)
        check(out_f64(y), r, rabs, out, accum, k // 128, f"wide fprop {m}x{n}x{k} mode={mode} out={out} accum={accum}")
    dY = inputs.random_bf16(135, (512, 8152), sd=1e-3)
    X2 = inputs.random_bf16(136, (512, 2008))
    qdt, sdt, _, wqdt, wsdt, _ = quant_both(hip, orc, dY, "col", mode)
    qxt, sxt, _, wqxt, wsxt, _ = quant_both(hip, orc, X2, "col", mode)
    dw = hip.linear_wgrad(qdt, sdt, qxt, sxt, out, accum=accum)
    r, rabs = full(orc, wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
    check(out_f64(dw), r, rabs, out, accum, 4, f"wide wgrad 8152x2008x512 mode={mode} out={out} accum={accum}")


@ACCUMS_POW2
def test_exact_special_cases(hip, orc, accum):
    """Bit-exact GPU results where the arithmetic is exact: A = identity with
    power-of-two block scales gives the dequantised B^T; small integers with
    unit scales give the integer product."""
    rng = np.random.default_rng(5)
    table = orc.decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    K = N = 256
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = 0x38
    sa = np.ones((K // 128, K), np.float32)
    b = rng.choice(finite, (N, K))
    sbk = (2.0 ** rng.integers(-20, 20, (N // 128, K // 128))).astype(np.float32)
    y = hip.fp8_gemm_blockscaled(dev(a), dev(sa), dev(b), dev(sbk), 0, sbk.shape[1], 1, 1, accum=accum)
    np.testing.assert_array_equal(out_f64(y), orc.gemm(a, sa, b, sbk, 0, sbk.shape[1], 1))
    ints = {int(v): c for c, v in enumerate(table) if not np.isnan(v) and v == int(v) and abs(v) <= 8 and c != 0x80}
    keys = np.array(sorted(ints))
    M, N, K = 200, 136, 768
    ia, ib = rng.choice(keys, (M, K)), rng.choice(keys, (N, K))
    ca = np.vectorize(ints.get)(ia).astype(np.uint8)
    cb = np.vectorize(ints.get)(ib).astype(np.uint8)
    y = hip.fp8_gemm_blockscaled(dev(ca), dev(np.ones((K // 128, M), np.float32)), dev(cb),
                                 dev(np.ones((2, K // 128), np.float32)), 0, K // 128, 1, 1, accum=accum)
    np.testing.assert_array_equal(out_f64(y), (ia @ ib.T).astype(np.float64))


@ACCUMS
def test_empty_k_and_deterministic(hip, orc, accum):
    """K = 0 writes zeros; repeated calls are bitwise identical."""
    M, N = 130, 140
    a = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((1, M), dtype=torch.float32, device="cuda")
    sb = torch.zeros((2, 1), dtype=torch.float32, device="cuda")
    d = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    hip.fp8_gemm_blockscaled(a, sa, b, sb, 0, 1, 1, 1, d=d, accum=accum)
    assert torch.count_nonzero(d).item() == 0
    X = inputs.random_bf16(9, (512, 2048))
    W = inputs.random_bf16(10, (384, 2048), sd=0.02, outliers=False)
    qx, sx = hip.fp8_quant_tile(dev_bf16(X))
    qw, sw, _ = hip.fp8_quant_block(dev_bf16(W))
    y1 = hip.linear_fprop(qx, sx, qw, sw, 1, accum=accum)
    y2 = hip.linear_fprop(qx, sx, qw, sw, 1, accum=accum)
    assert torch.equal(y1, y2)


@ACCUMS_POW2
@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_large_k_split(hip, orc, mode, accum):
    """256x256x65536 with U(-1,1) inputs (workload 4b): split-K partials
    reduced in a fixed order, fp32 output, bitwise repeatable."""
    if accum == 2 and mode == 0:
        pytest.skip("the scaled-MFMA mode takes power-of-two scales only")
    d = workload("large_k")
    qa, sa, _, wqa, wsa, _ = quant_both(hip, orc, d["A"], "row", mode)
    qb, sb, _, wqb, wsb, _ = quant_both(hip, orc, d["B"], "block", mode)
    assert hip.gemm_workspace_bytes(256, 256, 65536) > 0
    y = hip.linear_fprop(qa, sa, qb, sb, 1, accum=accum)
    y2 = hip.linear_fprop(qa, sa, qb, sb, 1, accum=accum)
    assert torch.equal(y, y2)
    r, rabs = full(orc, wqa, wsa, wqb, wsb, 0, wsb.shape[1], 1)
    log(f"large K mode={mode} accum={accum}: normwise {oracle.normwise_err(out_f64(y), r):.3e}")
    check(out_f64(y), r, rabs, 1, accum, 512, f"large K mode={mode} accum={accum}")




@pytest.mark.parametrize("K", [4096, 65536])
def test_promotion_benefit_large_k(hip, orc, K):
    """What per-128 promotion buys: the large-K workload's U(-1,1) operands
    (M = N = 256; the first 4096 columns for K = 4096) on the GPU in all three
    modes, beside the oracle's model of a 14-bit accumulator that is never
    promoted and one promoted every 128 elements (32 products per exact
    chunk, on the output's first 32 x 128 block).  Every GPU mode must meet
    the fp32 gate on the full output and stay at least 10x below the
    never-promoted model's error on the block."""
    d = workload("large_k")
    A, B = np.ascontiguousarray(d["A"][:, :K]), np.ascontiguousarray(d["B"][:, :K])
    rows = []
    for mode, accums in ((0, (0, 1)), (1, (2,))):
        qa, sa, _, wqa, wsa, _ = quant_both(hip, orc, A, "row", mode)
        qb, sb, _, wqb, wsb, _ = quant_both(hip, orc, B, "block", mode)
        r, rabs = full(orc, wqa, wsa, wqb, wsb, 0, wsb.shape[1], 1)
        blk = (slice(0, 32), slice(0, 128))
        ra, sa32, rb = wqa[:32], np.ascontiguousarray(wsa[:, :32]), wqb[:128]
        sb128 = np.ascontiguousarray(wsb[:1])
        for name, interval in (("model never promoted", 0), ("model promoted every 128", 128)):
            y = orc.gemm_limited(ra, sa32, rb, sb128, 0, sb128.shape[1], 1, 14, 32, interval)
            m = oracle.measure(y, r[blk], None, 1, K // 128)
            rows.append((f"{name} (scales {'pow2' if mode else 'fp32'})", m["normwise"], m["elementwise"]))
        unpromoted = rows[-2][1]
        for accum in accums:
            y = out_f64(hip.linear_fprop(qa, sa, qb, sb, 1, accum=accum))
            check(y, r, rabs, 1, accum, K // 128, f"K={K} scales={'pow2' if mode else 'fp32'} accum={accum}")
            mb = oracle.measure(y[blk], r[blk], None, 1, K // 128)
            rows.append((f"GPU accum={accum}", mb["normwise"], mb["elementwise"]))
            assert mb["normwise"] * 10 <= unpromoted, (accum, mb, unpromoted)
    for name, nw, el in rows:
        log(f"K={K} {name}: normwise {nw:.2e}, elementwise {el:.2e} (32 x 128 block)")


@functools.lru_cache(maxsize=2)
def _dense_fprop_reference(mode):
    """The oracle's full result for workload 1 (every one of the 75.5M
    outputs; about 30 s on 16 host threads) and R_abs, for FP32 (mode 0) or
    power-of-two (mode 1) scales, computed once per session."""
    d = workload("dense_fprop")
    orc = oracle.default()
    wqx, wsx = orc.quant_tile(d["X"], 0, mode)
    wqw, wsw, _ = orc.quant_block(d["W"], mode)
    r, rabs = full(orc, wqx, wsx, wqw, wsw, 0, wsw.shape[1], 1)
    return wqx, wsx, wqw, wsw, r, rabs


@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
def test_wgrad_224_column_tiles(hip, orc, out):
    """Per-column-scale GEMMs (Wgrad) in the FP32-scale FP8 mode on shapes
    whose launch on a 256-CU MI355X takes 256 x 224 tiles (one round of 256
    of them, against 224 wide tiles): dW[2000x7104] over 256 tokens (a last
    row tile of 208 rows, a last column tile of 160 columns) and dW[1800x7168]
    over 384 tokens (a last row tile of 8 rows); every output compared."""
    for i, (T, Nw, C) in enumerate([(256, 2000, 7104), (384, 1800, 7168)]):
        dY = inputs.random_bf16(161 + 2 * i, (T, Nw), sd=1e-3)
        X = inputs.random_bf16(162 + 2 * i, (T, C))
        qdt, sdt, _, wqdt, wsdt, _ = quant_both(hip, orc, dY, "col", 0)
        qxt, sxt, _, wqxt, wsxt, _ = quant_both(hip, orc, X, "col", 0)
        dw = hip.linear_wgrad(qdt, sdt, qxt, sxt, out, accum=1)
        r, rabs = full(orc, wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
        check(out_f64(dw), r, rabs, out, 1, T // 128, f"wgrad 224-column tiles {Nw}x{C}x{T} out={out}")


@pytest.mark.parametrize("accum", [1, 2], ids=["mfma8", "mfma8pow2"])
def test_group_counts_mixed_tiles(hip, orc, accum):
    """K = 128 .. 896 (one to seven K groups: the single-group path, odd
    counts, even counts and the steady K loop of the FP8 modes' kernels) on
    X[4000x896] W[4200x896], a shape whose launch on a 256-CU MI355X puts
    columns 0..2303 on 256 x 256 tiles and the rest on 256 x 128 tiles, the
    last row and column of tiles partial.  The GEMMs run on K-prefixes of
    the quantised operands (row strides 896); the rows of the first, a
    middle and the last row of tiles are compared on every column."""
    mode = 1 if accum == 2 else 0
    M, N, KMAX = 4000, 4200, 896
    X = inputs.random_bf16(151, (M, KMAX))
    W = inputs.random_bf16(152, (N, KMAX), sd=0.02, outliers=False)
    qx, sx, _, wqx, wsx, _ = quant_both(hip, orc, X, "row", mode)
    qw, sw, _, wqw, wsw, _ = quant_both(hip, orc, W, "block", mode)
    rows = np.r_[0:64, 1984:2048, 3904:4000]
    for g in range(1, KMAX // 128 + 1):
        K = 128 * g
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        hip.fp8_gemm_blockscaled(qx[:, :K], sx[:g], qw[:, :K], sw[:, :g], hip.BSCALE_BLOCK, sw.stride(0), 1, 0, d=y,
                                 accum=accum)
        a = np.ascontiguousarray(wqx[rows, :K])
        sa = np.ascontiguousarray(wsx[:g, rows])
        b = np.ascontiguousarray(wqw[:, :K])
        sb = np.ascontiguousarray(wsw[:, :g])
        r, rabs = full(orc, a, sa, b, sb, 0, sb.shape[1], 1)
        check(out_f64(y)[rows], r, rabs, 0, accum, g, f"mixed tiles {M}x{N}x{K} accum={accum}")


@ACCUMS_POW2
def test_dense_fprop_full_size(hip, orc, accum):
    """Workload 1 at its real size (4096 x 18432 x 7168, bf16 out) in the
    launch configuration the benchmark times -- FP32 scales for the exact and
    FP8-matrix-core modes, power-of-two scales for the mode that applies them
    inside the MFMA -- every output against the oracle."""
    mode = 1 if accum == 2 else 0
    d = workload("dense_fprop")
    qx, sx, _, _, _, _ = quant_both(hip, orc, d["X"], "row", mode)
    qw, sw, _, _, _, _ = quant_both(hip, orc, d["W"], "block", mode)
    y = hip.linear_fprop(qx, sx, qw, sw, 0, accum=accum)
    _, _, _, _, r, rabs = _dense_fprop_reference(mode)
    check(out_f64(y), r, rabs, 0, accum, 56, f"dense fprop full size scales={'pow2' if mode else 'fp32'} accum={accum}")


@functools.lru_cache(maxsize=1)
def _expert_backward_reference():
    """The oracle's full Dgrad and Wgrad of workload 2 with their
    absolute-value companions, computed once per session."""
    d = workload("expert_backward")
    orc = oracle.default()
    wqd, wsd = orc.quant_tile(d["dY"], 0, 0)
    _, wsw, wqwt = orc.quant_block(d["W"], 0, transpose=True)
    dgrad = full(orc, wqd, wsd, wqwt, wsw, 0, 1, wsw.shape[1])
    wqdt, wsdt = orc.quant_tile(d["dY"], 1, 0)
    wqxt, wsxt = orc.quant_tile(d["X"], 1, 0)
    wgrad = full(orc, wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
    return dgrad, wgrad


@ACCUMS
def test_expert_backward_full_size(hip, orc, accum):
    """Workload 2 at its real size: Dgrad 8192x7168x2048 and Wgrad
    2048x7168x8192, fp32 out, every output against the oracle."""
    d = workload("expert_backward")
    (r, rabs), (rw, rwabs) = _expert_backward_reference()
    qd, sd_, _, _, _, _ = quant_both(hip, orc, d["dY"], "row", 0)
    qw, sw, qwt, _, _, _ = quant_both(hip, orc, d["W"], "block", 0)
    dx = hip.linear_dgrad(qd, sd_, qwt, sw, 1, accum=accum)
    check(out_f64(dx), r, rabs, 1, accum, 16, f"expert dgrad full size accum={accum}")
    del dx
    qdt, sdt, _, _, _, _ = quant_both(hip, orc, d["dY"], "col", 0)
    qxt, sxt, _, _, _, _ = quant_both(hip, orc, d["X"], "col", 0)
    dw = hip.linear_wgrad(qdt, sdt, qxt, sxt, 1, accum=accum)
    check(out_f64(dw), rw, rwabs, 1, accum, 64, f"expert wgrad full size accum={accum}")


@ACCUMS_POW2
@pytest.mark.parametrize("kind", [0, 1], ids=["block", "tile"])
@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_gemm_fused_quant(hip, orc, mode, kind, accum):
    """The GEMM with its output quantised 1x128 in the epilogue equals the
    GEMM's bf16 output quantised by fp8_quant_tile, and that quantisation of
    the bf16 output equals the oracle's, bit for bit: ragged M (300 rows),
    N = 384, K = 1024, both B-scale kinds."""
    if accum == 2 and mode == 0:
        pytest.skip("the scaled-MFMA mode takes power-of-two scales only")
    X = inputs.random_bf16(111, (300, 1024))
    qx, sx = hip.fp8_quant_tile(dev_bf16(X), hip.AXIS_ROW, mode)
    if kind == 0:
        W = inputs.random_bf16(112, (384, 1024), sd=0.02, outliers=False)
        qw, sw, _ = hip.fp8_quant_block(dev_bf16(W), mode)
        s0, s1 = sw.shape[1], 1
    else:
        # per-column B scales: quantise W^T in 128x1 groups along K
        W = inputs.random_bf16(112, (1024, 384), sd=0.02, outliers=False)
        qw, sw = hip.fp8_quant_tile(dev_bf16(W), hip.AXIS_COL, mode)
        s0, s1 = sw.shape[1], 0
    q, s = hip.fp8_gemm_blockscaled_quant(qx, sx, qw, sw, kind, s0, s1, mode, accum=accum)
    y = hip.fp8_gemm_blockscaled(qx, sx, qw, sw, kind, s0, s1, hip.OUT_BF16, accum=accum)
    q2, s2 = hip.fp8_quant_tile(y, hip.AXIS_ROW, mode)
    assert torch.equal(q, q2) and torch.equal(s, s2)
    wq, ws = orc.quant_tile(host(y), 0, mode)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s), ws)


@ACCUMS_POW2
def test_gemm_fused_quant_full_size(hip, orc, accum):
    """Dense Fprop at its real size with the output quantised 1x128 in the
    epilogue, on the launches each mode takes (256 x 256 tiles with two
    128-column images per tile in the FP8-matrix-core modes): every code and
    scale equals the oracle's quantisation of the same GEMM's bf16 output,
    and the separate quantiser's (two passes on the GPU)."""
    mode = 1 if accum == 2 else 0
    d = workload("dense_fprop")
    qx, sx = hip.fp8_quant_tile(dev_bf16(d["X"]), hip.AXIS_ROW, mode)
    qw, sw, _ = hip.fp8_quant_block(dev_bf16(d["W"]), mode)
    q, s = hip.fp8_gemm_blockscaled_quant(qx, sx, qw, sw, 0, sw.shape[1], 1, mode, accum=accum)
    y = hip.linear_fprop(qx, sx, qw, sw, hip.OUT_BF16, accum=accum)
    wq, ws = orc.quant_tile(host(y), 0, mode)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))
    q2, s2 = hip.fp8_quant_tile(y, hip.AXIS_ROW, mode)
    assert torch.equal(q, q2) and torch.equal(s, s2)
    log(f"fused quant full size accum={accum}: {wq.size} codes and {ws.size} scales equal the oracle's")


@ACCUMS_POW2
def test_strided_operands_and_output(hip, orc, accum):
    """Operands read through leading dimensions larger than K and outputs
    written into a wider matrix give the same bits as the contiguous call
    and leave the bytes outside the view alone; shapes include one row, one
    K group and a ragged N (M = 1, 129; K = 128, 640; N = 136)."""
    rng = np.random.default_rng(17)
    table = orc.decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    for M, K in [(1, 128), (129, 640)]:
        N = 136
        a = rng.choice(finite, (M, K))
        b = rng.choice(finite, (N, K))
        sa = (2.0 ** rng.integers(-4, 4, (K // 128, M))).astype(np.float32)
        sb = (2.0 ** rng.integers(-4, 4, ((N + 127) // 128, K // 128))).astype(np.float32)
        ref = hip.fp8_gemm_blockscaled(dev(a), dev(sa), dev(b), dev(sb), 0, K // 128, 1, 1, accum=accum)
        A = torch.zeros((M, K + 144), dtype=torch.uint8, device="cuda")
        A[:, 16:16 + K] = dev(a)
        B = torch.zeros((N, K + 32), dtype=torch.uint8, device="cuda")
        B[:, :K] = dev(b)
        SA = torch.zeros((K // 128, M + 7), dtype=torch.float32, device="cuda")
        SA[:, :M] = dev(sa)
        D = torch.full((M, N + 12), -3.0, dtype=torch.float32, device="cuda")
        hip.fp8_gemm_blockscaled(A[:, 16:16 + K], SA[:, :M], B[:, :K], dev(sb), 0, K // 128, 1, 1,
                                 d=D[:, 4:4 + N], accum=accum)
        assert torch.equal(D[:, 4:4 + N], ref)
        assert torch.all(D[:, :4] == -3.0).item() and torch.all(D[:, 4 + N:] == -3.0).item()
        r = orc.gemm(a, sa, b, sb, 0, K // 128, 1)
        rabs = orc.gemm_abs(a, sa, b, sb, 0, K // 128, 1)
        check(out_f64(ref), r, rabs, 1, accum, K // 128, f"strided M={M} K={K} accum={accum}")

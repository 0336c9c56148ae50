"""GPU grouped (MoE expert) GEMM against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_gemm_amd import inputs
from gpu_util import workload, bf16_f64, check, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu
ACCUMS = pytest.mark.parametrize("accum", [0, 1], ids=["acc32", "mfma8"])
ACCUMS_POW2 = pytest.mark.parametrize("accum", [0, 1, 2], ids=["acc32", "mfma8", "mfma8pow2"])


def out_f64(t):
    h = host(t)
    return bf16_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


def quant_experts(hip, orc, Xcat, W, mode):
    G, N, K = W.shape
    qx, sx = hip.fp8_quant_tile(dev_bf16(Xcat), hip.AXIS_ROW, mode)
    wqx, wsx = orc.quant_tile(Xcat, 0, mode)
    np.testing.assert_array_equal(host(qx), wqx)
    np.testing.assert_array_equal(host(sx), wsx)
    qw, sw, _ = hip.fp8_quant_block(dev_bf16(W.reshape(G * N, K)), mode)
    wqw, wsw, _ = orc.quant_block(W.reshape(G * N, K), mode)
    np.testing.assert_array_equal(host(qw), wqw)
    np.testing.assert_array_equal(host(sw), wsw)
    return (qx, sx, qw.view(G, N, K), sw.view(G, N // 128, K // 128),
            wqx, wsx, wqw.reshape(G, N, K), wsw.reshape(G, N // 128, K // 128))


@ACCUMS_POW2
@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
def test_grouped_small_with_empty_experts(hip, orc, out, accum):
    """6 experts with 0, 1, 130, 0, 257 and 40 rows (empty experts, a single
    row, ragged tiles), N = 256, K = 512, power-of-two scales."""
    counts = [0, 1, 130, 0, 257, 40]
    offsets = np.zeros(len(counts) + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    Xcat = inputs.random_bf16(201, (int(offsets[-1]), 512))
    W = inputs.random_bf16(202, (len(counts), 256, 512), sd=0.02, outliers=False)
    qx, sx, qw, sw, wqx, wsx, wqw, wsw = quant_experts(hip, orc, Xcat, W, 1)
    y = hip.fp8_grouped_gemm(dev(offsets), qx, sx, qw, sw, out, accum=accum)
    r = orc.grouped_gemm(offsets, wqx, wsx, wqw, wsw)
    rabs = orc.grouped_gemm_abs(offsets, wqx, wsx, wqw, wsw)
    for e in range(len(counts)):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            check(out_f64(y)[r0:r1], r[r0:r1], rabs[r0:r1], out, accum, 4, f"expert {e} out={out} accum={accum}")


@pytest.mark.parametrize("accum", [1, 2], ids=["mfma8", "mfma8pow2"])
@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_grouped_short_k(hip, orc, K, accum):
    """Fewer K groups than the row tiles' pipeline depth (1, 2, 3 and 5
    groups): experts of 128, 64, 0, 17 and 129 rows (full, partial and empty
    128-row tiles, one just past them), N = 384, fp32 out."""
    counts = [128, 64, 0, 17, 129]
    offsets = np.zeros(len(counts) + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    Xcat = inputs.random_bf16(205 + K, (int(offsets[-1]), K))
    W = inputs.random_bf16(206 + K, (len(counts), 384, K), sd=0.02, outliers=False)
    qx, sx, qw, sw, wqx, wsx, wqw, wsw = quant_experts(hip, orc, Xcat, W, 1)
    y = hip.fp8_grouped_gemm(dev(offsets), qx, sx, qw, sw, 1, accum=accum)
    r = orc.grouped_gemm(offsets, wqx, wsx, wqw, wsw)
    rabs = orc.grouped_gemm_abs(offsets, wqx, wsx, wqw, wsw)
    check(out_f64(y), r, rabs, 1, accum, K // 128, f"short K={K} accum={accum}")


@pytest.mark.parametrize("accum", [1, 2], ids=["mfma8", "mfma8pow2"])
@pytest.mark.parametrize("out", [1, 0], ids=["f32", "bf16"])
def test_grouped_row_tile_boundaries(hip, orc, out, accum):
    """Experts on each side of every row-tile size the FP8 kernels choose
    (64, 128, 192, 256 rows), none, a few, and more than one 256-row tile
    (300 and 520 rows: a last tile of 44 and of 8 rows), N = 384, K = 640
    (five K groups: the three- and four-stage pipelines' tails), every
    output against the oracle."""
    counts = [64, 65, 128, 129, 192, 193, 256, 0, 7, 520, 300]
    offsets = np.zeros(len(counts) + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    Xcat = inputs.random_bf16(207, (int(offsets[-1]), 640))
    W = inputs.random_bf16(208, (len(counts), 384, 640), sd=0.02, outliers=False)
    qx, sx, qw, sw, wqx, wsx, wqw, wsw = quant_experts(hip, orc, Xcat, W, 1)
    y = hip.fp8_grouped_gemm(dev(offsets), qx, sx, qw, sw, out, accum=accum)
    r = orc.grouped_gemm(offsets, wqx, wsx, wqw, wsw)
    rabs = orc.grouped_gemm_abs(offsets, wqx, wsx, wqw, wsw)
    for e in range(len(counts)):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            check(out_f64(y)[r0:r1], r[r0:r1], rabs[r0:r1], out, accum, 5,
                  f"expert {e} ({counts[e]} rows) out={out} accum={accum}")


@ACCUMS_POW2
def test_grouped_strided_column_scales(hip, orc, accum):
    """The strided grouped GEMM with per-column B scales (tile kind): each
    expert's B[N x K] quantised in 1x128 groups along K, scales [K/128][N];
    experts of 0, 70, 200 and 300 rows, N = 256, K = 384, power-of-two
    scales, fp32 out, every output against the oracle."""
    counts = [0, 70, 200, 300]
    G, N, K = len(counts), 256, 384
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    Xcat = inputs.random_bf16(209, (int(offsets[-1]), K))
    Bw = inputs.random_bf16(210, (G * N, K), sd=0.02, outliers=False)
    qx, sx = hip.fp8_quant_tile(dev_bf16(Xcat), hip.AXIS_ROW, 1)
    wqx, wsx = orc.quant_tile(Xcat, 0, 1)
    qb = torch.empty((G * N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((G, K // 128, N), dtype=torch.float32, device="cuda")
    wq, ws = [], []
    for e in range(G):
        hip.fp8_quant_tile(dev_bf16(Bw[e * N:(e + 1) * N]), hip.AXIS_ROW, 1, q=qb[e * N:(e + 1) * N], s=sb[e])
        q_e, s_e = orc.quant_tile(Bw[e * N:(e + 1) * N], 0, 1)
        np.testing.assert_array_equal(host(qb[e * N:(e + 1) * N]), q_e)
        wq.append(q_e)
        ws.append(s_e)
    y = hip.fp8_grouped_gemm_strided(dev(offsets), qx, sx, G, N, qb, K, N * K, sb, hip.BSCALE_TILE, N, 0,
                                     (K // 128) * N, 1, accum=accum)
    got = out_f64(y)
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        a, sa = wqx[r0:r1], np.ascontiguousarray(wsx[:, r0:r1])
        r = orc.gemm(a, sa, wq[e], ws[e], 1, N, 0)
        rabs = orc.gemm_abs(a, sa, wq[e], ws[e], 1, N, 0)
        check(got[r0:r1], r, rabs, 1, accum, K // 128, f"strided tile-kind expert {e} accum={accum}")


@ACCUMS_POW2
def test_grouped_empty_k(hip, orc, accum):
    """K = 0: every routed row's output is the empty sum, zero, in every
    row-tile shape (experts of 70, 0, 300 and 150 rows); rows past
    offsets[G] keep their contents."""
    counts = [70, 0, 300, 150]
    G, N = len(counts), 256
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    rows = int(offsets[-1])
    a = torch.zeros((rows + 10, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((1, rows + 10), dtype=torch.float32, device="cuda")
    b = torch.zeros((G, N, 0), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((G, N // 128, 1), dtype=torch.float32, device="cuda")
    d = torch.full((rows + 10, N), 7.0, dtype=torch.float32, device="cuda")
    hip.fp8_grouped_gemm(dev(offsets), a, sa, b, sb, 1, rows_bound=rows + 10, d=d, accum=accum)
    assert torch.count_nonzero(d[:rows]).item() == 0
    assert torch.all(d[rows:] == 7.0).item()


@pytest.mark.parametrize("accum", [0, 1], ids=["acc32", "mfma8"])
def test_grouped_rows_beyond_offsets_untouched(hip, orc, accum):
    """Rows past offsets[G] (rows_bound larger than the routed rows) are not
    written."""
    offsets = np.array([0, 100, 160], np.int32)
    Xcat = inputs.random_bf16(203, (200, 256))
    W = inputs.random_bf16(204, (2, 128, 256), sd=0.02, outliers=False)
    qx, sx, qw, sw, *_ = quant_experts(hip, orc, Xcat, W, 0)
    d = torch.full((200, 128), 3.0, dtype=torch.float32, device="cuda")
    hip.fp8_grouped_gemm(dev(offsets), qx, sx, qw, sw, 1, rows_bound=200, d=d, accum=accum)
    assert torch.all(d[160:] == 3.0).item()




def _check_full(hip, orc, data, mode, tag, accum):
    Xcat, W, offsets = data["Xcat"], data["W"], data["offsets"]
    qx, sx, qw, sw, wqx, wsx, wqw, wsw = quant_experts(hip, orc, Xcat, W, mode)
    y = hip.fp8_grouped_gemm(dev(offsets), qx, sx, qw, sw, 0, accum=accum)
    r = orc.grouped_gemm(offsets, wqx, wsx, wqw, wsw)
    rabs = orc.grouped_gemm_abs(offsets, wqx, wsx, wqw, wsw)
    check(out_f64(y), r, rabs, 0, accum, wqw.shape[2] // 128, f"{tag} accum={accum}")


@ACCUMS_POW2
def test_grouped_upproj_full_size(hip, orc, accum):
    """Workload 3: 32 local experts of a top-8-of-256 routing of 4096
    tokens, N = 4096, K = 7168, power-of-two scales, bf16 out, every output
    against the oracle."""
    _check_full(hip, orc, workload("grouped_upproj"), 1, "grouped up-proj", accum)


@ACCUMS
def test_decode_grouped_full_size(hip, orc, accum):
    """Workload 4a: 64 experts with 1..256 rows each, N = 2048, K = 7168,
    every output against the oracle."""
    _check_full(hip, orc, workload("decode_grouped"), 0, "decode grouped", accum)


def _moe_dgrad_case(hip, orc, dY, W, offsets, accum, tag, sample=None):
    """M-grouped Dgrad dX_e = dY_e W_e through the strided grouped GEMM,
    reading the transposed copy of the stacked weight quantisation; the
    oracle is the dense oracle GEMM per expert on the same codes."""
    G, Nw, Kw = W.shape
    qd, sd = hip.fp8_quant_tile(dev_bf16(dY), hip.AXIS_ROW, 0)
    wqd, wsd = orc.quant_tile(dY, 0, 0)
    np.testing.assert_array_equal(host(qd), wqd)
    _, sw, qwt = hip.fp8_quant_block(dev_bf16(W.reshape(G * Nw, Kw)), 0, transpose=True)
    _, wsw, wqwt = orc.quant_block(W.reshape(G * Nw, Kw), 0, transpose=True)
    np.testing.assert_array_equal(host(qwt), wqwt)
    dx = hip.moe_dgrad(dev(offsets), qd, sd, qwt, sw, G, out_dtype=1, accum=accum)
    y = out_f64(dx)
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        a, sa = wqd[r0:r1], np.ascontiguousarray(wsd[:, r0:r1])
        b = np.ascontiguousarray(wqwt[:, e * Nw:(e + 1) * Nw])
        sbe = np.ascontiguousarray(wsw[e * Nw // 128:(e + 1) * Nw // 128])
        if sample is None:
            r = orc.gemm(a, sa, b, sbe, 0, 1, sbe.shape[1])
            rabs = orc.gemm_abs(a, sa, b, sbe, 0, 1, sbe.shape[1])
            got = y[r0:r1]
        else:
            rng = np.random.default_rng(e)
            mi, ni = rng.integers(0, r1 - r0, sample), rng.integers(0, Kw, sample)
            r = orc.gemm_entries(a, sa, b, sbe, 0, 1, sbe.shape[1], mi, ni)
            rabs = orc.gemm_abs_entries(a, sa, b, sbe, 0, 1, sbe.shape[1], mi, ni)
            got = y[r0:r1][mi, ni]
        check(got, r, rabs, 1, accum, Nw // 128, f"{tag} expert {e}")


@ACCUMS
def test_moe_dgrad_small(hip, orc, accum):
    """6 experts with 0, 1, 130, 0, 257 and 40 rows, N_w = 256, K_w = 384
    (ragged tiles, empty experts), fp32 out, every output compared."""
    counts = [0, 1, 130, 0, 257, 40]
    offsets = np.zeros(len(counts) + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    dY = inputs.random_bf16(211, (int(offsets[-1]), 256), sd=1e-3)
    W = inputs.random_bf16(212, (len(counts), 256, 384), sd=0.02, outliers=False)
    _moe_dgrad_case(hip, orc, dY, W, offsets, accum, f"moe dgrad small accum={accum}")


@ACCUMS
def test_moe_dgrad_upproj_full_size(hip, orc, accum):
    """Dgrad of the grouped up-projection at its real size: 32 experts,
    W_e[4096 x 7168], dY[rows x 4096] N(0,1e-3) with outliers, every output
    compared."""
    data = workload("grouped_upproj")
    offsets = data["offsets"]
    dY = inputs.random_bf16(213, (int(offsets[-1]), 4096), sd=1e-3)
    _moe_dgrad_case(hip, orc, dY, data["W"], offsets, accum, f"moe dgrad up-proj accum={accum}")


def _padded(counts):
    starts, p = [], 0
    for n in counts:
        starts.append(p)
        p += (n + 127) // 128 * 128
    return starts, p


@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_quant_grouped_col_small(hip, orc, mode):
    """128x1 groups per expert (0, 1, 130, 0, 257, 40 tokens; 200 columns,
    a ragged column tile): codes, padding and scales bit-exact."""
    counts = [0, 1, 130, 0, 257, 40]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = inputs.random_bf16(221, (int(offsets[-1]), 200))
    q, s = hip.fp8_quant_tile_grouped_col(dev_bf16(x), dev(offsets), mode)
    wq, ws = orc.quant_tile_grouped_col(x, offsets, mode)
    tp = wq.shape[1]
    np.testing.assert_array_equal(host(q)[:, :tp], wq)
    np.testing.assert_array_equal(host(s)[:tp // 128], ws)


@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
def test_quant_grouped_col_upproj_full_size(hip, orc, mode):
    """128x1 groups per expert at the up-projection's real size: dY[rows x
    4096] and X[rows x 7168] of the 32 experts (as the MoE Wgrad quantises
    them), every code, padding byte and scale bit-exact."""
    data = workload("grouped_upproj")
    offsets = data["offsets"]
    dY = inputs.random_bf16(224, (int(offsets[-1]), 4096), sd=1e-3)
    for name, x in (("dY", dY), ("X", data["Xcat"])):
        q, s = hip.fp8_quant_tile_grouped_col(dev_bf16(x), dev(offsets), mode)
        wq, ws = orc.quant_tile_grouped_col(x, offsets, mode)
        tp = wq.shape[1]
        np.testing.assert_array_equal(host(q)[:, :tp], wq)
        np.testing.assert_array_equal(host(s)[:tp // 128].view(np.uint32), ws.view(np.uint32))
        log(f"grouped 128x1 {name}[{x.shape[0]}x{x.shape[1]}] mode={mode}: {wq.size} codes bit-exact")


def _moe_wgrad_check(hip, orc, dY, X, offsets, accum, tag, sample=None, mode=0):
    counts = np.diff(offsets)
    dw = hip.moe_wgrad(dev(offsets), dev_bf16(dY), dev_bf16(X), mode, out_dtype=1, accum=accum)
    wqd, wsd = orc.quant_tile_grouped_col(dY, offsets, mode)
    wqx, wsx = orc.quant_tile_grouped_col(X, offsets, mode)
    starts, _ = _padded(counts)
    N, C = dY.shape[1], X.shape[1]
    for e, n in enumerate(counts):
        if n == 0:
            assert torch.count_nonzero(dw[e]).item() == 0
            continue
        k0, k1 = starts[e], starts[e] + (int(n) + 127) // 128 * 128
        a, sa = np.ascontiguousarray(wqd[:, k0:k1]), np.ascontiguousarray(wsd[k0 // 128:k1 // 128])
        b, sb = np.ascontiguousarray(wqx[:, k0:k1]), np.ascontiguousarray(wsx[k0 // 128:k1 // 128])
        if sample is None:
            r = orc.gemm(a, sa, b, sb, 1, sb.shape[1], 0)
            rabs = orc.gemm_abs(a, sa, b, sb, 1, sb.shape[1], 0)
            got = host(dw[e]).astype(np.float64)
        else:
            rng = np.random.default_rng(e)
            mi, ni = rng.integers(0, N, sample), rng.integers(0, C, sample)
            r = orc.gemm_entries(a, sa, b, sb, 1, sb.shape[1], 0, mi, ni)
            rabs = orc.gemm_abs_entries(a, sa, b, sb, 1, sb.shape[1], 0, mi, ni)
            got = dw[e][torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy().astype(np.float64)
        check(got, r, rabs, 1, accum, (k1 - k0) // 128, f"{tag} expert {e}")


@ACCUMS
def test_moe_wgrad_small(hip, orc, accum):
    """K-grouped Wgrad dW_e = dY_e^T X_e over ragged experts (0, 1, 130, 0,
    257, 40 tokens), N = 256, C = 200: every output compared; experts
    without tokens give zeros."""
    counts = [0, 1, 130, 0, 257, 40]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dY = inputs.random_bf16(222, (int(offsets[-1]), 256), sd=1e-3)
    X = inputs.random_bf16(223, (int(offsets[-1]), 200))
    _moe_wgrad_check(hip, orc, dY, X, offsets, accum, f"moe wgrad small accum={accum}")


@ACCUMS_POW2
def test_moe_wgrad_token_tails(hip, orc, accum):
    """Experts whose last 128-token group holds 31, 32, 33, 64, 65, 96, 97,
    128, 1, 63 and 127 tokens (every count of 32-token blocks the FP8 paths
    stage for it), N = 256, C = 384; power-of-two scales for the mode that
    needs them."""
    counts = [31, 32, 33, 64, 65, 96, 97, 128, 129, 191, 255]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dY = inputs.random_bf16(224, (int(offsets[-1]), 256), sd=1e-3)
    X = inputs.random_bf16(225, (int(offsets[-1]), 384))
    _moe_wgrad_check(hip, orc, dY, X, offsets, accum, f"moe wgrad tails accum={accum}", mode=int(accum == 2))


@ACCUMS
def test_moe_wgrad_upproj_full_size(hip, orc, accum):
    """Wgrad of the grouped up-projection experts at their real size: 32
    experts, dY[rows x 4096], X[rows x 7168] gathered per route, dW_e
    [4096 x 7168] fp32, every output compared."""
    data = workload("grouped_upproj")
    offsets = data["offsets"]
    dY = inputs.random_bf16(224, (int(offsets[-1]), 4096), sd=1e-3)
    _moe_wgrad_check(hip, orc, dY, data["Xcat"], offsets, accum, f"moe wgrad up-proj accum={accum}")

"""GPU backward re-tiling (1x128 codes -> 128x1 codes) against the CPU
oracle: codes and scales bit-exact, then the Wgrad GEMM on re-tiled
operands within the GEMM tolerance."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_gemm_amd import inputs
from gpu_util import check, workload, dev, dev_bf16, edge_rows, host, log

pytestmark = pytest.mark.gpu
MODES = pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])


def requant_both(hip, orc, q, s, mode):
    """Re-tile host codes/scales on the GPU and on the CPU; require
    bit-exact equality; return the GPU tensors."""
    qt, st = hip.fp8_requant_col(dev(q), dev(s), mode)
    wqt, wst = orc.requant_col(q, s, mode)
    np.testing.assert_array_equal(host(qt), wqt)
    np.testing.assert_array_equal(host(st).view(np.uint32), wst.view(np.uint32))
    return qt, st, wqt, wst


@pytest.mark.parametrize("mode_in", [0, 1], ids=["in_fp32", "in_pow2"])
@MODES
def test_requant_small(hip, orc, mode_in, mode):
    """256 x 384 with outliers, rows of extreme magnitude and the edge rows
    (zero groups, signed zeros, subnormals, ties, the bf16 maximum).  With
    power-of-two input scales the bf16-maximum row is replaced by 1e38: its
    scale rounds up to 2^120, and 256 * 2^120 -- the dequantised maximum --
    is not a finite fp32 (outside the contract)."""
    x = inputs.random_bf16(301, (256, 384))
    x[:9, :256] = edge_rows(256)
    if mode_in == 1:
        e = x[:9, :256]
        big = (e & 0x7FFF) == 0x7F7F
        e[big] = (e[big] & 0x8000) | 0x7E96  # +-0.997e38
    f = (np.random.default_rng(302).standard_normal((8, 384)) * 1e30).astype(np.float32)
    x[20:28] = (f.view(np.uint32) >> 16).astype(np.uint16)
    f = (np.random.default_rng(303).standard_normal((8, 384)) * 1e-30).astype(np.float32)
    x[40:48] = (f.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quant_tile(x, 0, mode_in)
    requant_both(hip, orc, q, s, mode)


@MODES
def test_requant_gpu_chain(hip, orc, mode):
    """The path as the backward pass runs it: X quantised 1x128 on the GPU in
    Fprop, re-tiled on the GPU for Wgrad."""
    x = inputs.random_bf16(304, (512, 640))
    q, s = hip.fp8_quant_tile(dev_bf16(x), hip.AXIS_ROW, mode)
    qt, st = hip.fp8_requant_col(q, s, mode)
    wq, ws = orc.quant_tile(x, 0, mode)
    wqt, wst = orc.requant_col(wq, ws, mode)
    np.testing.assert_array_equal(host(qt), wqt)
    np.testing.assert_array_equal(host(st), wst)


def test_requant_into_strided_outputs(hip, orc):
    """Leading dimensions larger than the matrix: only the addressed bytes
    change."""
    x = inputs.random_bf16(305, (256, 256))
    q, s = orc.quant_tile(x, 0, 0)
    qbig = torch.zeros((256, 320), dtype=torch.uint8, device="cuda")
    qbig[:, :256] = dev(q)
    sbig = torch.zeros((2, 272), dtype=torch.float32, device="cuda")
    sbig[:, :256] = dev(s)
    qt = torch.full((256, 288), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.full((2, 300), -1.0, dtype=torch.float32, device="cuda")
    hip.fp8_requant_col(qbig[:, :256], sbig[:, :256], 0, qt=qt[:, :256], st=st[:, :256])
    wqt, wst = orc.requant_col(q, s, 0)
    np.testing.assert_array_equal(host(qt)[:, :256], wqt)
    np.testing.assert_array_equal(host(st)[:, :256], wst)
    assert torch.all(qt[:, 256:] == 0xAB).item() and torch.all(st[:, 256:] == -1.0).item()


@pytest.mark.parametrize("accum", [0, 1], ids=["acc32", "mfma8"])
def test_requant_full_size_and_wgrad(hip, orc, accum):
    """Expert-backward X[8192 x 7168]: 1x128 codes from the forward pass
    re-tiled to 128x1 (all codes and scales compared), then Wgrad dW = dY^T X
    on the re-tiled operand, fp32 out, every output against the oracle."""
    d = workload("expert_backward")
    q, s = hip.fp8_quant_tile(dev_bf16(d["X"]), hip.AXIS_ROW, 0)
    wq, ws = orc.quant_tile(d["X"], 0, 0)
    np.testing.assert_array_equal(host(q), wq)
    qxt, sxt = hip.fp8_requant_col(q, s, 0)
    wqxt, wsxt = orc.requant_col(wq, ws, 0)
    np.testing.assert_array_equal(host(qxt), wqxt)
    np.testing.assert_array_equal(host(sxt), wsxt)
    qdt, sdt = hip.fp8_quant_tile(dev_bf16(d["dY"]), hip.AXIS_COL, 0)
    wqdt, wsdt = orc.quant_tile(d["dY"], 1, 0)
    np.testing.assert_array_equal(host(qdt), wqdt)
    dw = hip.linear_wgrad(qdt, sdt, qxt, sxt, 1, accum=accum)
    r = orc.gemm(wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
    rabs = orc.gemm_abs(wqdt, wsdt, wqxt, wsxt, 1, wsxt.shape[1], 0)
    check(host(dw).astype(np.float64), r, rabs, 1, accum, 64, f"wgrad on re-tiled X accum={accum}")


@MODES
def test_quant_dual_small(hip, orc, mode):
    """Both groupings from one read equal the two single-grouping oracle
    quantisations, on 256 x 384 with the edge rows and extreme magnitudes."""
    x = inputs.random_bf16(306, (256, 384), sd=1e-3)
    x[:9, :256] = edge_rows(256)
    f = (np.random.default_rng(307).standard_normal((8, 384)) * 1e35).astype(np.float32)
    x[100:108] = (f.view(np.uint32) >> 16).astype(np.uint16)
    qr, sr, qc, sc = hip.fp8_quant_dual(dev_bf16(x), mode)
    wqr, wsr = orc.quant_tile(x, 0, mode)
    wqc, wsc = orc.quant_tile(x, 1, mode)
    np.testing.assert_array_equal(host(qr), wqr)
    np.testing.assert_array_equal(host(sr), wsr)
    np.testing.assert_array_equal(host(qc), wqc)
    np.testing.assert_array_equal(host(sc), wsc)


def test_quant_dual_full_size(hip, orc):
    """Expert-backward dY[8192 x 2048], both groupings, all codes and scales."""
    d = workload("expert_backward")
    qr, sr, qc, sc = hip.fp8_quant_dual(dev_bf16(d["dY"]), 0)
    wqr, wsr = orc.quant_tile(d["dY"], 0, 0)
    wqc, wsc = orc.quant_tile(d["dY"], 1, 0)
    np.testing.assert_array_equal(host(qr), wqr)
    np.testing.assert_array_equal(host(sr), wsr)
    np.testing.assert_array_equal(host(qc), wqc)
    np.testing.assert_array_equal(host(sc), wsc)


def test_requant_every_code_round_trips(hip, orc):
    """Each column holds the 254 finite codes (in a different order per
    column) with unit row scales; the largest magnitude, 448, makes the new
    scale 1, so re-tiling must give back every code exactly -- the device
    decode of every finite code is exact."""
    table = orc.decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    rng = np.random.default_rng(9)
    q = np.zeros((256, 128), np.uint8)
    for c in range(128):
        q[:254, c] = rng.permutation(finite)
    s = np.ones((1, 256), np.float32)
    qt, st = hip.fp8_requant_col(dev(q), dev(s), 0)
    wqt, wst = orc.requant_col(q, s, 0)
    np.testing.assert_array_equal(host(qt), wqt)
    np.testing.assert_array_equal(host(st), wst)
    # the group holding 0x7E / 0xFE has scale 1: its codes come back unchanged
    for c in range(128):
        for g in range(2):
            if st[g, c] == 1.0:
                np.testing.assert_array_equal(host(qt)[c, 128 * g:128 * g + 128], q[128 * g:128 * g + 128, c])

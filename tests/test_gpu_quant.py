"""GPU quantisers against the CPU oracle: E4M3 codes and scales must match
bit for bit.  Runs through the C ABI (via the Python binding)."""
import numpy as np
import pytest
import torch

from block_scaled_gemm_amd import inputs
from gpu_util import workload, dev, dev_bf16, edge_rows, host, log

pytestmark = pytest.mark.gpu


def test_cast_all_fp32_patterns(hip, orc):
    """fp8_cast_e4m3 over every finite fp32 bit pattern equals the oracle's
    encoder (NaN / Inf patterns are outside the contract and skipped)."""
    chunk = 1 << 27
    bad = 0
    for start in range(0, 1 << 32, chunk):
        u = np.arange(start, start + chunk, dtype=np.uint32)
        f = u.view(np.float32)
        got = host(hip.fp8_cast_e4m3(dev(f)))
        want = orc.encode(f)
        finite = ((u >> 23) & 0xFF) != 0xFF
        mism = np.nonzero((got != want) & finite)[0]
        if mism.size:
            i = mism[0]
            log(f"cast mismatch at 0x{u[i]:08x}: gpu 0x{got[i]:02x} oracle 0x{want[i]:02x}")
        bad += mism.size
    assert bad == 0


def _row_case(name):
    if name == "tiny_X":
        return workload("tiny_fprop")["X"]
    if name == "tiny_W":
        return workload("tiny_fprop")["W"]
    if name == "edges":
        return edge_rows(512)
    if name == "ragged_rows":
        return inputs.random_bf16(5, (37, 384))
    if name == "dense_X":
        return workload("dense_fprop")["X"]
    raise KeyError(name)


@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
@pytest.mark.parametrize("case", ["tiny_X", "tiny_W", "edges", "ragged_rows", "dense_X"])
def test_quant_tile_row(hip, orc, case, mode):
    x = _row_case(case)
    log(f"quant_tile ROW {case} {x.shape} mode={mode}")
    q, s = hip.fp8_quant_tile(dev_bf16(x), hip.AXIS_ROW, mode)
    wq, ws = orc.quant_tile(x, 0, mode)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))


def _col_case(name):
    if name == "edges":
        return np.ascontiguousarray(edge_rows(256).T)  # [256, 9]: 9 columns, ragged
    if name == "ragged_cols":
        return inputs.random_bf16(6, (384, 200))
    if name == "dY":
        return workload("expert_backward")["dY"]
    if name == "X":
        return workload("expert_backward")["X"]
    raise KeyError(name)


@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
@pytest.mark.parametrize("case", ["edges", "ragged_cols", "dY", "X"])
def test_quant_tile_col(hip, orc, case, mode):
    x = _col_case(case)
    log(f"quant_tile COL {case} {x.shape} mode={mode}")
    # leading dimension padded to a multiple of 8 elements
    ld = (x.shape[1] + 7) // 8 * 8
    xp = np.zeros((x.shape[0], ld), np.uint16)
    xp[:, :x.shape[1]] = x
    q, s = hip.fp8_quant_tile(dev_bf16(xp)[:, :x.shape[1]], hip.AXIS_COL, mode)
    wq, ws = orc.quant_tile(x, 1, mode)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))


def _block_case(name):
    if name == "tiny_W":
        return workload("tiny_fprop")["W"]
    if name == "edges":
        return np.tile(edge_rows(256), (30, 1))  # 270 rows: ragged last block-row
    if name == "dense_W":
        return workload("dense_fprop")["W"]
    if name == "expert_W":
        return workload("expert_backward")["W"]
    if name == "odd_blocks":
        # five block columns: the last workgroup of a block row holds one block
        return inputs.random_bf16(9, (300, 640), sd=0.02)
    raise KeyError(name)


@pytest.mark.parametrize("mode", [0, 1], ids=["fp32", "pow2"])
@pytest.mark.parametrize("case", ["tiny_W", "edges", "odd_blocks", "expert_W", "dense_W"])
def test_quant_block(hip, orc, case, mode):
    w = _block_case(case)
    log(f"quant_block {case} {w.shape} mode={mode}")
    q, s, qt = hip.fp8_quant_block(dev_bf16(w), mode, transpose=True)
    wq, ws, wqt = orc.quant_block(w, mode, transpose=True)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(qt), wqt)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))


def test_quant_grouped_weights_pow2(hip, orc):
    """Every expert's weights of the grouped up-projection, stacked [G*N, K],
    in 128x128 blocks with power-of-two scales (blocks never straddle two
    experts because N is a multiple of 128)."""
    w = workload("grouped_upproj")["W"]
    G, N, K = w.shape
    log(f"quant_block grouped W {w.shape} pow2")
    flat = w.reshape(G * N, K)
    q, s, _ = hip.fp8_quant_block(dev_bf16(flat), 1)
    wq, ws, _ = orc.quant_block(flat, 1)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(s).view(np.uint32), ws.view(np.uint32))


def test_quant_into_strided_views(hip, orc):
    """Leading dimensions larger than the logical width are honoured and the
    padding is left untouched."""
    x = inputs.random_bf16(8, (64, 384))
    xp = np.zeros((64, 512), np.uint16)
    xp[:, :384] = x
    xd = dev_bf16(xp)[:, :384]
    qbuf = torch.full((64, 416), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((3, 80), -1.0, dtype=torch.float32, device="cuda")
    hip.fp8_quant_tile(xd, hip.AXIS_ROW, 0, q=qbuf[:, :384], s=sbuf[:, :64])
    wq, ws = orc.quant_tile(x, 0, 0)
    qh, sh = host(qbuf), host(sbuf)
    np.testing.assert_array_equal(qh[:, :384], wq)
    assert np.all(qh[:, 384:] == 0xAB)
    np.testing.assert_array_equal(sh[:, :64], ws)
    assert np.all(sh[:, 64:] == -1.0)

"""fp8_scales_are_pow2 on the GPU: the power-of-two quantisers' scales
pass; FP32 scales and planted non-powers (a mantissa, a sign, zero, a
denormal, inf, NaN) fail; strided views count only their entries; an
empty array passes; and with FP8BS_CHECK_POW2 set the power-of-two MFMA
mode refuses FP32 scales."""
import pytest
import torch

import block_scaled_gemm_amd as bs
from block_scaled_gemm_amd import inputs
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def test_quantiser_scales():
    X = dev_bf16(inputs.random_bf16(171, (512, 1024)))
    W = dev_bf16(inputs.random_bf16(172, (384, 1024), sd=0.02, outliers=False))
    _, s2 = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_POW2)
    _, sw2, _ = bs.fp8_quant_block(W, bs.SCALE_POW2)
    assert bs.scales_are_pow2(s2) and bs.scales_are_pow2(sw2)
    _, s1 = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32)
    _, sw1, _ = bs.fp8_quant_block(W, bs.SCALE_FP32)
    assert not bs.scales_are_pow2(s1) and not bs.scales_are_pow2(sw1)


@pytest.mark.parametrize("bad", [0.3, -0.25, 0.0, 2.0 ** -130, float("inf"), float("nan")],
                         ids=["mantissa", "negative", "zero", "denormal", "inf", "nan"])
def test_one_planted_entry_fails(bad):
    s = torch.full((8, 300), 0.25, dtype=torch.float32, device="cuda")
    assert bs.scales_are_pow2(s)
    s[5, 123] = bad
    assert not bs.scales_are_pow2(s)


def test_strided_views_and_empty():
    s = torch.full((8, 300), 2.0 ** -20, dtype=torch.float32, device="cuda")
    s[:, 1::2] = 0.3
    assert not bs.scales_are_pow2(s)
    assert bs.scales_are_pow2(s[:, ::2])         # a view: only its entries
    assert bs.scales_are_pow2(s, 8, 150, 300, 2)  # the same, as explicit strides
    assert not bs.scales_are_pow2(s, 8, 150, 300, 1)
    assert bs.scales_are_pow2(s, 0, 5, 300, 1)    # empty
    assert bs.scales_are_pow2(s, 1, 1, 0, 0)      # one entry, s[0]


def test_check_gate_of_the_pow2_mode(monkeypatch):
    X = dev_bf16(inputs.random_bf16(173, (256, 512)))
    W = dev_bf16(inputs.random_bf16(174, (256, 512), sd=0.02, outliers=False))
    qx, sx = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_FP32)
    qw, sw, _ = bs.fp8_quant_block(W, bs.SCALE_FP32)
    qx2, sx2 = bs.fp8_quant_tile(X, bs.AXIS_ROW, bs.SCALE_POW2)
    qw2, sw2, _ = bs.fp8_quant_block(W, bs.SCALE_POW2)
    monkeypatch.setenv("FP8BS_CHECK_POW2", "1")
    with pytest.raises(ValueError, match="powers of two"):
        bs.fp8_gemm_blockscaled(qx, sx, qw, sw, bs.BSCALE_BLOCK, sw.stride(0), 1, accum=bs.ACCUM_MFMA8_POW2)
    y = bs.fp8_gemm_blockscaled(qx2, sx2, qw2, sw2, bs.BSCALE_BLOCK, sw2.stride(0), 1, accum=bs.ACCUM_MFMA8_POW2)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all().item()
    # the FP32 modes are not gated
    bs.fp8_gemm_blockscaled(qx, sx, qw, sw, bs.BSCALE_BLOCK, sw.stride(0), 1, accum=bs.ACCUM_MFMA8)

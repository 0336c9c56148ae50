"""The allocation-free GEMM entry point (fp8_gemm_blockscaled_noalloc),
called through the C ABI, against fp8_gemm_blockscaled on the same inputs:
the same kernels and split count, so the outputs must be identical bit for
bit.  Two calls in a row, the second smaller, so a stale partial left in the
shared scratch array by the first call would show."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_f64, check, dev_bf16, host, log, workload

pytestmark = pytest.mark.gpu


def _pair(hip, A, B, accum, mode, out):
    """(output of fp8_gemm_blockscaled, output of the no-alloc call) for
    A[M x K] times B[N x K]^T; the no-alloc output starts filled with 7."""
    qa, sa = hip.fp8_quant_tile(dev_bf16(A), hip.AXIS_ROW, mode)
    qb, sb, _ = hip.fp8_quant_block(dev_bf16(B), mode)
    ref = hip.fp8_gemm_blockscaled(qa, sa, qb, sb, hip.BSCALE_BLOCK, sb.shape[1], 1, out, accum=accum)
    d = torch.full_like(ref, 7.0)
    hip.fp8_gemm_blockscaled_noalloc(qa, sa, qb, sb, hip.BSCALE_BLOCK, sb.shape[1], 1, d, out, accum=accum)
    torch.cuda.synchronize()
    return ref, d


@pytest.mark.parametrize("accum", [0, 1, 2], ids=["acc32", "mfma8", "mfma8pow2"])
def test_noalloc_matches_gemm_twice(hip, orc, accum):
    mode = 1 if accum == 2 else 0
    d = workload("large_k")
    # first call: 256 x 256 x 65536, whose 64 split-K partials fill the
    # whole 16 MiB scratch array
    M, N, K = 256, 256, 65536
    assert hip.gemm_workspace_bytes(M, N, K) == hip.NOALLOC_SCRATCH_BYTES
    log(f"no-alloc accum={accum}: call 1, {M}x{N}x{K}")
    ref, got = _pair(hip, d["A"], d["B"], accum, mode, hip.OUT_F32)
    assert torch.equal(got, ref)
    # second call: smaller and ragged, 200 x 136 x 16384 (16 splits, a
    # different partial layout over the same array)
    M, N, K = 200, 136, 16384
    A, B = np.ascontiguousarray(d["A"][:M, :K]), np.ascontiguousarray(d["B"][:N, :K])
    assert 0 < hip.gemm_workspace_bytes(M, N, K) < hip.NOALLOC_SCRATCH_BYTES
    log(f"no-alloc accum={accum}: call 2, {M}x{N}x{K}")
    ref2, got2 = _pair(hip, A, B, accum, mode, hip.OUT_F32)
    assert torch.equal(got2, ref2)
    wqa, wsa = orc.quant_tile(A, 0, mode)
    wqb, wsb, _ = orc.quant_block(B, mode)
    r = orc.gemm(wqa, wsa, wqb, wsb, 0, wsb.shape[1], 1)
    rabs = orc.gemm_abs(wqa, wsa, wqb, wsb, 0, wsb.shape[1], 1)
    check(host(got2).astype(np.float64), r, rabs, 1, accum, K // 128, f"no-alloc call 2 accum={accum}")


def test_noalloc_without_split(hip, orc):
    """A shape that needs no scratch (300 x 384 x 1024, bf16 out) goes
    straight through, identical to fp8_gemm_blockscaled."""
    A = workload("tiny_fprop")["X"]
    X = np.tile(A, (3, 2))[:300, :1024]
    W = np.tile(workload("tiny_fprop")["W"], (2, 2))[:384, :1024]
    assert hip.gemm_workspace_bytes(300, 384, 1024) == 0
    ref, got = _pair(hip, X, W, 1, 0, hip.OUT_BF16)
    assert torch.equal(got, ref)


def test_noalloc_rejects_oversize(hip):
    """More split-K partials than the array holds: refused, output untouched."""
    M, N, K = 512, 256, 65536
    a = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.ones((K // 128, M), dtype=torch.float32, device="cuda")
    sb = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    d = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(hip.FP8BSError) as e:
        hip.fp8_gemm_blockscaled_noalloc(a, sa, b, sb, 0, K // 128, 1, d, hip.OUT_F32)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(d == 3.0).item()

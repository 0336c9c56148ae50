"""What promotion every 128 elements buys at large K, on the oracle's model
of limited accumulation (CPU only).

The pages: FP8 GEMM on their tensor cores keeps about 14 bits while it
accumulates ([cameseeing-1171527], passage on accumulation precision), a
K = 4096 test reached a relative error of nearly 2% ([qna-131281], passage
on the preliminary test), and copying partial sums to FP32 registers every
128 elements fixes it ([why-be-59061], passage on the 128-element interval).
The model (oracle.gemm_limited, pinned on hand-worked cases in
tests/golden/limited_accumulation.txt): 32 products (one instruction's K
for FP8 on that hardware) are added exactly, then the running sum is cut to
14 significant bits.  Inputs: the large-K workload's U(-1, 1) operands,
quantised 1x128 and 128x128 with FP32 scales; a 32 x 128 block of the output
at K = 4096 (the first 4096 columns) and K = 65536."""
import functools

import numpy as np
import pytest

import oracle
from block_scaled_gemm_amd import inputs

BITS, CHUNK = 14, 32


@functools.lru_cache(maxsize=1)
def errors():
    orc = oracle.default()
    d = inputs.large_k()
    out = {}
    for K in (4096, 65536):
        A, B = d["A"][:32, :K], d["B"][:128, :K]
        qa, sa = orc.quant_tile(A, 0, 0)
        qb, sb, _ = orc.quant_block(B, 0)
        r = orc.gemm(qa, sa, qb, sb, 0, sb.shape[1], 1)
        row = {}
        for name, chunk, interval in (("unpromoted", CHUNK, 0), ("promoted", CHUNK, 128),
                                      ("unpromoted_chunk4", 4, 0), ("promoted_chunk4", 4, 128)):
            y = orc.gemm_limited(qa, sa, qb, sb, 0, sb.shape[1], 1, BITS, chunk, interval)
            row[name] = oracle.measure(y, r, None, 1, K // 128)
        out[K] = row
    for K, row in out.items():
        print(f"K={K}: " + "; ".join(f"{n} normwise {m['normwise']:.2e} elementwise {m['elementwise']:.2e}"
                                     for n, m in row.items()))
    return out


def test_promoted_error_stays_small_at_any_k():
    e = errors()
    for K in (4096, 65536):
        assert e[K]["promoted"]["normwise"] <= 1e-3, (K, e[K]["promoted"])
    # the promoted error does not grow with K (each group starts from zero)
    assert e[65536]["promoted"]["normwise"] <= 2 * e[4096]["promoted"]["normwise"]


def test_unpromoted_error_grows_with_k():
    e = errors()
    for K in (4096, 65536):
        assert e[K]["unpromoted"]["normwise"] > 1e-3, (K, e[K]["unpromoted"])
        assert e[K]["unpromoted"]["normwise"] > 10 * e[K]["promoted"]["normwise"]
    assert e[65536]["unpromoted"]["normwise"] > 4 * e[4096]["unpromoted"]["normwise"]


@pytest.mark.parametrize("K", [4096, 65536])
def test_finer_chunks_lose_more(K):
    """Cutting after every 4 products instead of 32 loses more (the size of
    the pages' reported error, percent level at K = 4096, sits between the
    two); promotion keeps both below the fp32 gate."""
    e = errors()[K]
    assert e["unpromoted_chunk4"]["normwise"] > e["unpromoted"]["normwise"]
    assert e["promoted_chunk4"]["normwise"] <= 1e-3

"""Helpers for the GPU parity tests: host <-> device moves, cached workload
inputs, the edge-case inputs and the one gate every GEMM test applies
(the comparator itself lives in oracle/compare.py).  No method arithmetic
here."""
import functools
import sys

import numpy as np
import torch


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(y, r, rabs, out, accum, groups, tag):
    """Gate a GPU GEMM output y (float64 values) against the oracle's r with
    the comparator of oracle/compare.py, logging every measure."""
    import oracle
    ok, why, m = oracle.gate(y, r, rabs, out, accum, groups)
    log(f"{tag}: {oracle.describe(m, out)}")
    assert ok, (tag, why, m)


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    a = np.ascontiguousarray(bits, np.uint16).view(np.int16)
    return torch.from_numpy(a).to("cuda").view(torch.bfloat16)


def dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def edge_rows(cols=256):
    """Rows of bf16 bits whose 128-element groups exercise the edge cases:
    all zero, signed zeros, bf16 subnormals only, exact ties after a
    power-of-two scale, the largest bf16, the smallest normal, a single
    outlier, and alternating signs."""
    assert cols % 128 == 0
    rows = []
    f = lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    z = np.zeros(cols, np.float32)
    rows.append(f(z))                                   # all zero
    r = z.copy(); r[::2] = -0.0; rows.append(f(r))      # signed zeros
    r = np.full(cols, 2.0 ** -130, np.float32); r[1::3] = -(2.0 ** -133); rows.append(f(r))  # subnormals
    r = np.zeros(cols, np.float32)
    r[0::128] = 448.0; r[1::128] = 17.0; r[2::128] = 19.0; r[3::128] = 1.5 * 2 ** -9
    r[4::128] = 2.0 ** -10; r[5::128] = -(2.0 ** -10); r[6::128] = 232.0; r[7::128] = -3.25
    rows.append(f(r))                                   # ties (pow2 scale 1)
    r = np.full(cols, 3.3895314e38, np.float32); r[1::2] *= -1; rows.append(f(r))  # max bf16
    r = np.full(cols, 2.0 ** -126, np.float32); rows.append(f(r))  # min normal
    r = np.full(cols, 1e-3, np.float32); r[77] = 1e4; r[200 % cols] = -5e3; rows.append(f(r))  # outlier
    r = np.linspace(-7, 7, cols).astype(np.float32); rows.append(f(r))
    r = np.linspace(-1e-30, 3e-31, cols).astype(np.float32); rows.append(f(r))
    return np.stack(rows)


# The workload inputs are large; generate each once per test session (the
# arrays are shared, so tests must not modify them).
_cache = functools.lru_cache(maxsize=None)


@_cache
def workload(name):
    from block_scaled_gemm_amd import inputs
    return {"tiny_fprop": inputs.tiny_fprop, "dense_fprop": inputs.dense_fprop,
            "expert_backward": inputs.expert_backward, "grouped_upproj": inputs.grouped_upproj,
            "decode_grouped": inputs.decode_grouped, "large_k": inputs.large_k}[name]()

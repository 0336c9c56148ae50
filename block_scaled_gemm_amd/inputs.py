"""Seeded synthetic inputs shaped like the fine-grained FP8 linear's workloads.

This module draws random numbers and rounds them to bf16; it holds none of
the quantisation or GEMM arithmetic.  Tests, the benchmark and the smoke
check feed the same arrays to the HIP library and to the CPU oracle.

Recipe (all on the host, numpy only):
  * generator for workload i: ``numpy.random.Generator(PCG64(SeedSequence(1000 + i)))``
    split with ``SeedSequence.spawn`` into one child stream per tensor, in
    the order each builder lists;
  * "N(0, sd)" draws float32 standard normals and multiplies by sd (sd is a
    standard deviation);
  * "with outliers" multiplies an independent Bernoulli(0.001) subset of the
    entries by 100 (positions drawn as geometric gaps from the tensor's own
    stream), in float32, before the single rounding;
  * every tensor is rounded once from float32 to bf16, round-half-even, and
    returned as its uint16 bit pattern.
"""
import numpy as np

OUTLIER_RATE = 1e-3
OUTLIER_GAIN = 100.0
_CHUNK = 1 << 24  # elements per generation chunk (bounds the float32 temp)


def bf16_bits(f32):
    """Round float32 values to bf16 (half to even); return uint16 bits.
    Inputs here are finite."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bits -> float32 values (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def streams(workload, n):
    """n independent child generators for workload index `workload`."""
    children = np.random.SeedSequence(1000 + workload).spawn(n)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def _outlier_positions(rng, n):
    """Sorted positions of a Bernoulli(OUTLIER_RATE) subset of range(n)."""
    pos = []
    at = -1
    while True:
        gaps = rng.geometric(OUTLIER_RATE, size=max(16, int(n * OUTLIER_RATE * 1.2) + 16))
        steps = at + np.cumsum(gaps)
        keep = steps[steps < n]
        pos.append(keep)
        if keep.size < steps.size:
            break
        at = int(steps[-1])
    return np.concatenate(pos).astype(np.int64)


def normal_bf16(rng, shape, sd, outliers):
    """bf16 bits of N(0, sd) draws, optionally with x100 outliers."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, np.uint16)
    pos = _outlier_positions(rng, n) if outliers else None
    p = 0
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        f = rng.standard_normal(stop - start, dtype=np.float32)
        f *= np.float32(sd)
        if outliers:
            q = p
            while q < pos.size and pos[q] < stop:
                q += 1
            f[pos[p:q] - start] *= np.float32(OUTLIER_GAIN)
            p = q
        out[start:stop] = bf16_bits(f)
    return out.reshape(shape)


def uniform_bf16(rng, shape, lo, hi):
    """bf16 bits of U(lo, hi) draws."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        f = rng.uniform(lo, hi, size=stop - start).astype(np.float32)
        out[start:stop] = bf16_bits(f)
    return out.reshape(shape)


# ---- the five workloads ---------------------------------------------------------

def tiny_fprop():
    """Workload 0: X[128x512] N(0,1) with outliers, W[256x512] N(0,0.02)."""
    gx, gw = streams(0, 2)
    return {"X": normal_bf16(gx, (128, 512), 1.0, True),
            "W": normal_bf16(gw, (256, 512), 0.02, False)}


def dense_fprop():
    """Workload 1: X[4096x7168] N(0,1) with outliers, W[18432x7168] N(0,0.02)."""
    gx, gw = streams(1, 2)
    return {"X": normal_bf16(gx, (4096, 7168), 1.0, True),
            "W": normal_bf16(gw, (18432, 7168), 0.02, False)}


def expert_backward():
    """Workload 2: dY[8192x2048] N(0,1e-3) with outliers, X[8192x7168] N(0,1)
    with outliers, W[2048x7168] N(0,0.02)."""
    gd, gx, gw = streams(2, 3)
    return {"dY": normal_bf16(gd, (8192, 2048), 1e-3, True),
            "X": normal_bf16(gx, (8192, 7168), 1.0, True),
            "W": normal_bf16(gw, (2048, 7168), 0.02, False)}


def topk_routing(rng, tokens, experts, topk):
    """Each token picks `topk` distinct experts uniformly at random.
    Returns an int32 [tokens, topk] array."""
    keys = rng.random((tokens, experts))
    return np.argsort(keys, axis=1, kind="stable")[:, :topk].astype(np.int32)


def gather_by_expert(choice, local_experts):
    """Token lists per local expert (token order kept) and the offsets."""
    rows = []
    counts = []
    for e in range(local_experts):
        toks = np.nonzero((choice == e).any(axis=1))[0]
        rows.append(toks)
        counts.append(toks.size)
    offsets = np.zeros(local_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return np.concatenate(rows).astype(np.int64), offsets


def grouped_upproj(K=7168, N=4096, local=32, tokens=4096, experts=256, topk=8,
                   weights=True):
    """Workload 3: 4096 tokens routed top-8 of 256 experts; this GPU holds
    experts 0..31.  X[4096xK] N(0,1) with outliers is gathered per route;
    W[32, N, K] N(0,0.02)."""
    gr, gx, gw = streams(3, 3)
    choice = topk_routing(gr, tokens, experts, topk)
    tok, offsets = gather_by_expert(choice, local)
    X = normal_bf16(gx, (tokens, K), 1.0, True)
    out = {"offsets": offsets, "tokens": tok, "Xcat": X[tok]}
    if weights:
        out["W"] = normal_bf16(gw, (local, N, K), 0.02, False)
    return out


def decode_grouped(K=7168, N=2048, G=64, weights=True):
    """Workload 4a: 64 experts with U{1..256} rows each, X N(0,1) with
    outliers, W[64, N, K] N(0,0.02)."""
    gs, gx, gw, _, _ = streams(4, 5)
    counts = gs.integers(1, 257, size=G)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    out = {"offsets": offsets,
           "Xcat": normal_bf16(gx, (int(offsets[-1]), K), 1.0, True)}
    if weights:
        out["W"] = normal_bf16(gw, (G, N, K), 0.02, False)
    return out


def large_k(M=256, N=256, K=65536):
    """Workload 4b: A[MxK], B[NxK] U(-1, 1)."""
    _, _, _, ga, gb = streams(4, 5)
    return {"A": uniform_bf16(ga, (M, K), -1.0, 1.0),
            "B": uniform_bf16(gb, (N, K), -1.0, 1.0)}


def random_bf16(seed, shape, sd=1.0, outliers=True):
    """Ad-hoc seeded tensor for tests at other sizes (same recipe)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return normal_bf16(rng, shape, sd, outliers)

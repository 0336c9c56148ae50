"""The comparator: how a block-scaled GEMM output is measured against the
oracle's result, and the gate it has to pass.

TEST INFRASTRUCTURE, like the rest of oracle/: only tests/,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.
Pure numpy; it computes no GEMM itself (the oracle's ``gemm`` and
``gemm_abs`` give R and R_abs).

The pages quote a "maximum relative error" of nearly 2% for a K = 4096 FP8
GEMM whose tensor cores accumulate with limited precision
([qna-131281], passage on the preliminary accuracy test) without defining
it, and the tolerances this path is held to (1e-3 for fp32 output, 8e-3 for
bf16) are stated in the same words.  Three measures are computed for an
output y (float64 values) against the oracle's fp64 result R:

  normwise     max|y - R| / max|R|
               the largest error relative to the output's overall size;
  elementwise  max over elements of |y - R| / max(|R|, 0.01 * max|R|)
               the per-element relative error, its denominator floored at 1%
               of the largest |R| (a plain per-element ratio is unbounded
               where an output is near zero); this is the stricter of the
               two and the one every exact-partials result is held to;
  bound ratio  max over elements of |y - R| / B, with
               B = 2^-10 * R_abs + groups * 2^-23 * R_abs + u_out * |R|
               where R_abs is the same GEMM over the absolute values of the
               codes (scales are positive) and u_out = 2^-8 (bf16 output) or
               2^-23 (fp32): the error contract of group partials formed on
               the FP8 matrix cores, whose sum inside one instruction keeps
               about 2^-12 of the largest product, plus one fp32 rounding per
               group and the output's own rounding.

Gate (``gate``):
  exact group partials (accum 0): elementwise <= tol and normwise <= tol;
  FP8 matrix-core partials (accum 1, 2): normwise <= tol and bound ratio
      <= 1; their elementwise figure is reported, not gated (on some
      workloads it is above tol: the matrix cores' limited sum inside each
      group is what the pages' scheme accepts, and the per-element floor at
      1% of max|R| is tighter than that sum's error on small outputs).
tol = 8e-3 for bf16 output, 1e-3 for fp32.
"""
import numpy as np

OUT_BF16, OUT_F32 = 0, 1
TOL = {OUT_BF16: 8e-3, OUT_F32: 1e-3}
FLOOR_FRAC = 1e-2
# error terms of the FP8-matrix-core contract (see the module docstring)
MFMA_SUM_LOSS = 2.0 ** -10
GROUP_ROUND = 2.0 ** -23
OUT_ROUND = {OUT_BF16: 2.0 ** -8, OUT_F32: 2.0 ** -23}


def _f64(a):
    return np.asarray(a, np.float64)


def normwise_err(y, r):
    """max|y - r| / max|r| over the whole output.  An all-zero r gives 0
    when y is all zero too and inf otherwise."""
    y, r = _f64(y), _f64(r)
    if r.size == 0:
        return 0.0
    diff = float(np.max(np.abs(y - r)))
    top = float(np.max(np.abs(r)))
    if top == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / top


def max_rel_err(y, r, floor_frac=FLOOR_FRAC):
    """max over elements of |y - r| / max(|r|, floor_frac * max|r|).  An
    all-zero r gives 0 when y is all zero too and inf otherwise."""
    y, r = _f64(y), _f64(r)
    if r.size == 0:
        return 0.0
    diff = np.abs(y - r)
    top = float(np.max(np.abs(r)))
    if top == 0.0:
        return 0.0 if float(np.max(diff)) == 0.0 else float("inf")
    den = np.maximum(np.abs(r), floor_frac * top)
    return float(np.max(diff / den))


def fp8_partials_bound(r, rabs, out_dtype, groups):
    """Per-element error bound B of FP8-matrix-core group partials (module
    docstring): 2^-10 * rabs + groups * 2^-23 * rabs + u_out * |r|."""
    r, rabs = _f64(r), _f64(rabs)
    return (MFMA_SUM_LOSS * rabs + groups * GROUP_ROUND * rabs
            + OUT_ROUND[out_dtype] * np.abs(r))


def bound_ratio(y, r, rabs, out_dtype, groups):
    """max |y - r| / B over the elements (0 for an empty output).  Where B
    is 0 (every product of the element is zero) the error must be 0 too:
    such an element contributes 0 when it is exact and inf otherwise."""
    y, r = _f64(y), _f64(r)
    if r.size == 0:
        return 0.0
    diff = np.abs(y - r)
    b = fp8_partials_bound(r, rabs, out_dtype, groups)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(b > 0, diff / np.where(b > 0, b, 1.0), np.where(diff > 0, np.inf, 0.0))
    return float(np.max(q))


def measure(y, r, rabs, out_dtype, groups):
    """All three measures of y against r: a dict with 'normwise',
    'elementwise' and 'bound_ratio' (None when rabs is None)."""
    m = {"normwise": normwise_err(y, r), "elementwise": max_rel_err(y, r)}
    m["bound_ratio"] = None if rabs is None else bound_ratio(y, r, rabs, out_dtype, groups)
    return m


def passes(m, out_dtype, accum):
    """(ok, reason) of the gate for a result of ``measure``."""
    tol = TOL[out_dtype]
    if not m["normwise"] <= tol:
        return False, f"normwise {m['normwise']:.3e} > {tol:.0e}"
    if accum == 0:
        if not m["elementwise"] <= tol:
            return False, f"elementwise {m['elementwise']:.3e} > {tol:.0e}"
    else:
        if m["bound_ratio"] is None:
            return False, "FP8-matrix-core result without R_abs"
        if not m["bound_ratio"] <= 1.0:
            return False, f"error / bound {m['bound_ratio']:.3f} > 1"
    return True, "ok"


def gate(y, r, rabs, out_dtype, accum, groups):
    """``measure`` then ``passes``: returns (ok, reason, measures)."""
    m = measure(y, r, rabs, out_dtype, groups)
    ok, why = passes(m, out_dtype, accum)
    return ok, why, m


def describe(m, out_dtype):
    """One line of the measures, with the tolerance."""
    s = (f"normwise {m['normwise']:.3e}, elementwise {m['elementwise']:.3e} "
         f"(tol {TOL[out_dtype]:.0e})")
    if m.get("bound_ratio") is not None:
        s += f", error/bound {m['bound_ratio']:.3f}"
    return s

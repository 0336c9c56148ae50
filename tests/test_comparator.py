"""The comparator (oracle/compare.py) and R_abs, on the CPU.

Pins: each measure against values worked by hand.  Input mutations: an
output element, one code byte or one scale changed after the fact must be
reported by every measure and fail the gate in every accumulation mode.
Comparator mutations: plausible slips (a wrong denominator, a wrong axis, a
floor taken per element, the sign bits left in R_abs, a dropped bound term)
planted in copies of the comparator must each fail a pin."""
import types

import numpy as np
import pytest

import oracle
from oracle import compare as C
from block_scaled_gemm_amd import inputs


def real_comparator(orc):
    return types.SimpleNamespace(normwise_err=C.normwise_err, max_rel_err=C.max_rel_err,
                                 fp8_partials_bound=C.fp8_partials_bound, bound_ratio=C.bound_ratio,
                                 passes=C.passes, measure=C.measure, gemm_abs=orc.gemm_abs)


# ---- pins (each takes a comparator namespace) ------------------------------------

def pin_normwise_hand(cmp):
    """0.5 / 4.5 = 1/9: the largest error over the largest |R|."""
    y = np.array([[1.0, 2.0], [3.0, 4.0]])
    r = np.array([[1.0, 2.0], [3.0, 4.5]])
    assert abs(cmp.normwise_err(y, r) - 1.0 / 9.0) < 1e-15
    # a negative error counts by its size
    assert abs(cmp.normwise_err(-y, -r) - 1.0 / 9.0) < 1e-15
    y2 = r.copy()
    y2[0, 1] = 1.0  # error -1 against max|R| 4.5
    assert abs(cmp.normwise_err(y2, r) - 1.0 / 4.5) < 1e-15


def pin_normwise_whole_output(cmp):
    """The denominator is the largest |R| of the whole output, not of the
    element's row or column: 0.5 / 100."""
    r = np.array([[100.0, 1.0], [1.0, 1.0]])
    y = r.copy()
    y[1, 1] = 1.5
    assert abs(cmp.normwise_err(y, r) - 0.005) < 1e-15


def pin_elementwise_hand(cmp):
    """|y - R| / max(|R|, 0.01 max|R|), the largest over the elements."""
    # an exact zero output: denominator is the floor, 0.01 * 100 = 1
    r = np.array([[100.0, 0.5], [0.0, 1.0]])
    y = np.array([[100.0, 0.5], [0.5, 1.0]])
    assert abs(cmp.max_rel_err(y, r) - 0.5) < 1e-15
    # a small output above the floor uses its own size: 0.2 / 2
    r = np.array([[100.0, 2.0]])
    y = np.array([[100.0, 2.2]])
    assert abs(cmp.max_rel_err(y, r) - 0.1) < 1e-12
    # 1 / 50 beside a larger relative error elsewhere that is smaller in size
    r = np.array([[100.0, 50.0, 10.0]])
    y = np.array([[100.0, 51.0, 10.05]])
    assert abs(cmp.max_rel_err(y, r) - 0.02) < 1e-12
    # below the floor: 0.3 / (0.01 * 200) = 0.15, not 0.3 / 0.1
    r = np.array([[200.0, 0.1]])
    y = np.array([[200.0, 0.4]])
    assert abs(cmp.max_rel_err(y, r) - 0.15) < 1e-12


def pin_zero_reference(cmp):
    """An all-zero R: 0 when y is zero too, inf for any other y."""
    z = np.zeros((3, 4))
    assert cmp.normwise_err(z, z) == 0.0 and cmp.max_rel_err(z, z) == 0.0
    y = z.copy()
    y[2, 1] = 1e-30
    assert cmp.normwise_err(y, z) == np.inf and cmp.max_rel_err(y, z) == np.inf


def pin_bound_hand(cmp):
    """B = 2^-10 R_abs + groups 2^-23 R_abs + u_out |R|, with u_out 2^-23
    (fp32) or 2^-8 (bf16), worked out by hand."""
    b = cmp.fp8_partials_bound(np.array([[1.0]]), np.array([[3.0]]), 1, 2)
    # 3/1024 + 6/2^23 + 1/2^23
    assert b[0, 0] == 0.0029296875 + 7.0 / 8388608.0
    b = cmp.fp8_partials_bound(np.array([[-2.0]]), np.array([[2.0]]), 0, 1)
    # 2/1024 + 2/2^23 + 2/256 (|R|, not R)
    assert b[0, 0] == 0.001953125 + 2.0 / 8388608.0 + 0.0078125
    r = np.array([[1.0, 10.0]])
    rabs = np.array([[3.0, 10.0]])
    bb = 0.0029296875 + 7.0 / 8388608.0
    y = np.array([[1.0 + bb / 2, 10.0]])
    assert abs(cmp.bound_ratio(y, r, rabs, 1, 2) - 0.5) < 1e-12


def pin_bound_zero_products(cmp):
    """Where every product is zero (R_abs = 0) the bound is 0: an exact 0
    passes, anything else is an unbounded error."""
    r = np.zeros((1, 2))
    assert cmp.bound_ratio(r, r, r, 1, 4) == 0.0
    y = r.copy()
    y[0, 1] = 1e-30
    assert cmp.bound_ratio(y, r, r, 1, 4) == np.inf


def pin_rabs(cmp):
    """R_abs sums the products' sizes: codes 1 and -1 against 1 and 1 give
    R = 0 but R_abs = 2 (4 with a row scale of 2); R_abs is unchanged by
    flipping code signs and is never below |R|."""
    K = 128
    a = np.zeros((1, K), np.uint8)
    a[0, 0], a[0, 1] = 0x38, 0xB8
    b = np.zeros((1, K), np.uint8)
    b[0, 0], b[0, 1] = 0x38, 0x38
    ones = np.ones((1, 1), np.float32)
    assert oracle.gemm(a, ones, b, ones, 0, 1, 1)[0, 0] == 0.0
    assert cmp.gemm_abs(a, ones, b, ones, 0, 1, 1)[0, 0] == 2.0
    assert cmp.gemm_abs(a, 2 * ones, b, ones, 0, 1, 1)[0, 0] == 4.0
    rng = np.random.default_rng(3)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    a = rng.choice(codes, (9, 256))
    b = rng.choice(codes, (130, 256))
    sa = rng.uniform(0.5, 2, (2, 9)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (2, 2)).astype(np.float32)
    rabs = cmp.gemm_abs(a, sa, b, sb, 0, 2, 1)
    assert np.all(rabs >= np.abs(oracle.gemm(a, sa, b, sb, 0, 2, 1)))
    np.testing.assert_array_equal(cmp.gemm_abs(a ^ np.uint8(0x80), sa, b, sb, 0, 2, 1), rabs)


def pin_gate_rules(cmp):
    """The gate: exact partials need elementwise <= tol; FP8-matrix-core
    partials need the bound; every mode needs normwise <= tol."""
    ok = lambda m, out, acc: cmp.passes(m, out, acc)[0]
    m = {"normwise": 1e-3, "elementwise": 9e-3, "bound_ratio": 0.9}
    assert not ok(m, 0, 0) and ok(m, 0, 1) and ok(m, 0, 2)
    m = {"normwise": 1e-3, "elementwise": 7e-3, "bound_ratio": 1.1}
    assert ok(m, 0, 0) and not ok(m, 0, 1) and not ok(m, 0, 2)
    m = {"normwise": 2e-3, "elementwise": 2e-3, "bound_ratio": 0.5}
    assert ok(m, 0, 0) and not ok(m, 1, 0) and not ok(m, 1, 1)
    m = {"normwise": 5e-4, "elementwise": 5e-4, "bound_ratio": None}
    assert ok(m, 1, 0) and not ok(m, 1, 1)


PINS = [pin_normwise_hand, pin_normwise_whole_output, pin_elementwise_hand, pin_zero_reference,
        pin_bound_hand, pin_bound_zero_products, pin_rabs, pin_gate_rules]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_comparator_pin(orc, pin):
    pin(real_comparator(orc))


# ---- input mutations ------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    """The tiny Fprop workload quantised by the oracle, its exact result
    and R_abs; y0 is that result rounded once to fp32 (a correct output)."""
    orc = oracle.default()
    d = inputs.tiny_fprop()
    qx, sx = orc.quant_tile(d["X"], 0, 0)
    qw, sw, _ = orc.quant_block(d["W"], 0)
    r = orc.gemm(qx, sx, qw, sw, 0, sw.shape[1], 1)
    rabs = orc.gemm_abs(qx, sx, qw, sw, 0, sw.shape[1], 1)
    y0 = r.astype(np.float32).astype(np.float64)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, r=r, rabs=rabs, y0=y0, groups=qx.shape[1] // 128)


def _all_report(y, r, rabs, groups):
    m = C.measure(y, r, rabs, 1, groups)
    assert m["normwise"] > C.TOL[1], m
    assert m["elementwise"] > C.TOL[1], m
    assert m["bound_ratio"] > 1.0, m
    for accum in (0, 1, 2):
        assert not C.passes(m, 1, accum)[0], (accum, m)


def test_correct_output_passes(tiny):
    for accum in (0, 1, 2):
        ok, why, m = C.gate(tiny["y0"], tiny["r"], tiny["rabs"], 1, accum, tiny["groups"])
        assert ok, (accum, why)
    assert C.measure(tiny["y0"], tiny["r"], tiny["rabs"], 1, 4)["elementwise"] < 1e-6


def test_mutated_output_element_is_reported(tiny):
    r, rabs, g = tiny["r"], tiny["rabs"], tiny["groups"]
    b = C.fp8_partials_bound(r, rabs, 1, g)
    i = np.unravel_index(np.argmin(b), b.shape)
    y = tiny["y0"].copy()
    y[i] += max(10 * b[i], 0.01 * np.max(np.abs(r)))
    _all_report(y, r, rabs, g)


def test_mutated_code_byte_is_reported(orc, tiny):
    """One activation code's sign flipped (the largest code of row 3): the
    output computed from the original codes no longer matches the oracle's
    result for the codes it was given."""
    qx = tiny["qx"].copy()
    k = int(np.argmax(qx[3] & 0x7F))
    qx[3, k] ^= np.uint8(0x80)
    sw = tiny["sw"]
    r2 = orc.gemm(qx, tiny["sx"], tiny["qw"], sw, 0, sw.shape[1], 1)
    rabs2 = orc.gemm_abs(qx, tiny["sx"], tiny["qw"], sw, 0, sw.shape[1], 1)
    _all_report(tiny["y0"], r2, rabs2, tiny["groups"])


def test_mutated_scale_is_reported(orc, tiny):
    """One 1x128 scale doubled (row 5, group 1)."""
    sx = tiny["sx"].copy()
    sx[1, 5] *= 2
    sw = tiny["sw"]
    r2 = orc.gemm(tiny["qx"], sx, tiny["qw"], sw, 0, sw.shape[1], 1)
    rabs2 = orc.gemm_abs(tiny["qx"], sx, tiny["qw"], sw, 0, sw.shape[1], 1)
    _all_report(tiny["y0"], r2, rabs2, tiny["groups"])


def test_mutated_weight_scale_is_reported(orc, tiny):
    """One 128x128 block scale halved."""
    sw = tiny["sw"].copy()
    sw[1, 2] *= 0.5
    r2 = orc.gemm(tiny["qx"], tiny["sx"], tiny["qw"], sw, 0, sw.shape[1], 1)
    rabs2 = orc.gemm_abs(tiny["qx"], tiny["sx"], tiny["qw"], sw, 0, sw.shape[1], 1)
    _all_report(tiny["y0"], r2, rabs2, tiny["groups"])


# ---- comparator mutations ---------------------------------------------------------------

def _f(a):
    return np.asarray(a, np.float64)


def _mut_no_floor(y, r, floor_frac=C.FLOOR_FRAC):
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.nanmax(np.abs(_f(y) - _f(r)) / np.abs(_f(r))))


def _mut_floor_per_element(y, r, floor_frac=C.FLOOR_FRAC):
    d = np.maximum(np.abs(_f(r)), floor_frac * np.abs(_f(r)))
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.nanmax(np.abs(_f(y) - _f(r)) / d))


def _mut_normwise_per_row(y, r):
    y, r = _f(y), _f(r)
    top = np.max(np.abs(r), axis=-1, keepdims=True)
    return float(np.max(np.abs(y - r) / top))


def _mut_normwise_signed(y, r):
    y, r = _f(y), _f(r)
    return float(np.max(y - r) / np.max(np.abs(r)))


def _mut_normwise_mean(y, r):
    y, r = _f(y), _f(r)
    return float(np.max(np.abs(y - r)) / np.mean(np.abs(r)))


def _mut_bound_no_mfma_term(r, rabs, out_dtype, groups):
    return groups * C.GROUP_ROUND * _f(rabs) + C.OUT_ROUND[out_dtype] * np.abs(_f(r))


def _mut_bound_signed_r(r, rabs, out_dtype, groups):
    return C.MFMA_SUM_LOSS * _f(rabs) + groups * C.GROUP_ROUND * _f(rabs) + C.OUT_ROUND[out_dtype] * _f(r)


def _mut_gate_elementwise_never(m, out_dtype, accum):
    tol = C.TOL[out_dtype]
    if not m["normwise"] <= tol:
        return False, "normwise"
    if accum != 0 and (m["bound_ratio"] is None or m["bound_ratio"] > 1.0):
        return False, "bound"
    return True, "ok"


def _bound_ratio_with(bound_fn):
    def br(y, r, rabs, out_dtype, groups):
        d = np.abs(_f(y) - _f(r))
        b = bound_fn(r, rabs, out_dtype, groups)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(b > 0, d / np.where(b > 0, b, 1.0), np.where(d > 0, np.inf, 0.0))
        return float(np.max(q))
    return br


COMPARATOR_MUTATIONS = {
    "elementwise_floor_dropped": dict(max_rel_err=_mut_no_floor),
    "elementwise_floor_per_element": dict(max_rel_err=_mut_floor_per_element),
    "normwise_per_row": dict(normwise_err=_mut_normwise_per_row),
    "normwise_signed_error": dict(normwise_err=_mut_normwise_signed),
    "normwise_mean_denominator": dict(normwise_err=_mut_normwise_mean),
    "bound_without_mfma_term": dict(fp8_partials_bound=_mut_bound_no_mfma_term,
                                    bound_ratio=_bound_ratio_with(_mut_bound_no_mfma_term)),
    "bound_signed_r": dict(fp8_partials_bound=_mut_bound_signed_r,
                           bound_ratio=_bound_ratio_with(_mut_bound_signed_r)),
    "gate_ignores_elementwise": dict(passes=_mut_gate_elementwise_never),
}


def _rabs_sign_bits_kept(orc):
    # R_abs with the absolute value applied to the scales instead of the codes
    return lambda a, sa, b, sb, k, s0, s1: orc.gemm(a, np.abs(sa), b, np.abs(sb), k, s0, s1)


def _failing_pins(cmp):
    failed = []
    for pin in PINS:
        try:
            pin(cmp)
        except Exception:
            failed.append(pin.__name__)
    return failed


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # the slips divide by zero
@pytest.mark.parametrize("name", sorted(COMPARATOR_MUTATIONS) + ["rabs_sign_bits_kept"])
def test_comparator_mutation_is_caught(orc, name):
    cmp = real_comparator(orc)
    if name == "rabs_sign_bits_kept":
        cmp.gemm_abs = _rabs_sign_bits_kept(orc)
    else:
        for k, v in COMPARATOR_MUTATIONS[name].items():
            setattr(cmp, k, v)
    assert _failing_pins(cmp), f"no pin rejects the comparator slip {name}"


def test_unmutated_comparator_passes(orc):
    assert _failing_pins(real_comparator(orc)) == []

"""Checks that pin the CPU oracle to facts fixed outside it.

Each check takes an ``oracle.Oracle`` so the mutation tests can run the same
checks against deliberately broken builds of oracle.c.  Every check raises
AssertionError on failure.  None of them calls the HIP library.
"""
import ctypes
import fractions
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
BUILD = os.path.join(HERE, "pins", "_build")

_brute = None


def brute_lib():
    """tests/pins/e4m3_brute.c built with gcc (cached under pins/_build)."""
    global _brute
    if _brute is None:
        os.makedirs(BUILD, exist_ok=True)
        src = os.path.join(HERE, "pins", "e4m3_brute.c")
        out = os.path.join(BUILD, "libe4m3_brute.so")
        if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                            "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"],
                           check=True)
            os.replace(out + ".tmp", out)
        L = ctypes.CDLL(out)
        L.brute_check.restype = ctypes.c_int64
        L.brute_check.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.POINTER(ctypes.c_uint32),
                                  ctypes.POINTER(ctypes.c_uint8),
                                  ctypes.POINTER(ctypes.c_uint8)]
        L.brute_candidates.restype = None
        L.brute_candidates.argtypes = [ctypes.POINTER(ctypes.c_double)]
        _brute = L
    return _brute


def bf16_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_bf16_exact(values):
    """bf16 bits of float values that must be exactly representable."""
    f = np.asarray(values, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not a bf16"
    return (u >> 16).astype(np.uint16)


# ---- codec ----------------------------------------------------------------------

def check_codec_exhaustive(orc, stride=1, start=0):
    """Every finite fp32 bit pattern (or every stride-th one) encodes to the
    brute-force nearest E4M3 candidate, ties to the even code, saturating."""
    L = brute_lib()
    fn = ctypes.cast(orc.L.orc_e4m3_encode, ctypes.c_void_p)
    bad_bits = ctypes.c_uint32()
    got = ctypes.c_uint8()
    want = ctypes.c_uint8()
    bad = L.brute_check(fn, start, stride, ctypes.byref(bad_bits),
                        ctypes.byref(got), ctypes.byref(want))
    assert bad == 0, (f"{bad} fp32 patterns mis-encoded; first 0x{bad_bits.value:08x}"
                      f" -> 0x{got.value:02x}, brute force 0x{want.value:02x}")


def check_decode_table(orc):
    """decode() agrees with the brute-force candidate list, mirrored for the
    sign, with NaN only at 0x7F / 0xFF, and is strictly increasing on
    0x00..0x7E."""
    L = brute_lib()
    cand = (ctypes.c_double * 127)()
    L.brute_candidates(cand)
    cand = np.array(cand[:])
    t = orc.decode_table()
    assert np.all(np.diff(cand) > 0)
    np.testing.assert_array_equal(t[:127], cand)
    np.testing.assert_array_equal(t[128:255], -cand)
    assert np.isnan(t[127]) and np.isnan(t[255])
    assert np.signbit(t[128]) and t[128] == 0


def check_round_trip(orc):
    """encode(decode(c)) == c for every finite code (+0 and -0 kept apart)."""
    t = orc.decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = t[codes].astype(np.float32)
    np.testing.assert_array_equal(orc.encode(vals), codes)


def load_anchors():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_anchors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()[:2]
            out.append((int(code, 16), val))
    return out


def check_anchors(orc):
    t = orc.decode_table()
    for code, val in load_anchors():
        if val == "nan":
            assert np.isnan(t[code]), hex(code)
        elif val == "-0":
            assert t[code] == 0 and np.signbit(t[code]), hex(code)
        else:
            assert t[code] == float(fractions.Fraction(val)), (hex(code), val, t[code])
            if val != "0":
                assert orc.encode(np.float32(fractions.Fraction(val)))[()] == code


# ---- scale and quantisation -------------------------------------------------------

def _parse_scale(text):
    text = text.strip()
    if text.startswith("fp32("):
        num, den = text[5:-1].split("/")
        return np.float32(num) / np.float32(den)
    if text.startswith("2^"):
        return np.float32(2.0 ** int(text[2:]))
    return np.float32(fractions.Fraction(text))


def load_worked():
    stanzas = []
    cur = {}
    with open(os.path.join(GOLDEN, "quant_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    stanzas.append(cur)
                    cur = {}
                continue
            key, rest = line.split(None, 1)
            cur[key] = rest
    if cur:
        stanzas.append(cur)
    return stanzas


def check_worked_examples(orc):
    """The hand-worked groups of tests/golden/quant_worked.txt, as a 1x128
    row group, a 128x1 column group and (replicated) a 128x128 block."""
    ex = load_worked()
    assert len(ex) >= 5
    for st in ex:
        pow2 = st["mode"] == "pow2"
        vals = np.zeros(128, np.float32)
        for item in st["in"].split():
            i, v = item.split(":")
            vals[int(i)] = np.float32(float(v))
        bits = f32_bf16_exact(vals)
        want_codes = np.zeros(128, np.uint8)
        for item in st["out"].split():
            i, c = item.split(":")
            want_codes[int(i)] = int(c, 16)
        want_s = _parse_scale(st["s"])
        q, s = orc.quant_tile(bits.reshape(1, 128), 0, pow2)
        np.testing.assert_array_equal(q[0], want_codes, err_msg=str(st))
        assert s[0, 0] == want_s, (st, s[0, 0], want_s)
        q, s = orc.quant_tile(bits.reshape(128, 1), 1, pow2)
        np.testing.assert_array_equal(q[0], want_codes, err_msg=str(st))
        assert s[0, 0] == want_s
        blk = np.tile(bits, (128, 1))
        q, s, qt = orc.quant_block(blk, pow2, transpose=True)
        np.testing.assert_array_equal(q, np.tile(want_codes, (128, 1)))
        np.testing.assert_array_equal(qt, q.T)
        assert s[0, 0] == want_s


def brute_group(bits, pow2, table):
    """Independent brute force for one group of bf16 bits (see
    brute_group_f32)."""
    return brute_group_f32(bf16_f32(bits), pow2, table)


def brute_group_f32(x, pow2, table):
    """Independent brute force for one group of fp32 values: amax from the
    values, the scale by trying every power of two (POW2) or by the fp32
    quotient, and every code by scanning all 254 finite codes for the
    nearest value."""
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    floor_a = np.float32(448.0 * 2.0 ** -126)
    a = max(amax, floor_a)
    if pow2:
        k = min(k for k in range(-140, 140) if float(a) <= 448.0 * 2.0 ** k)
        s = np.float32(2.0 ** k)
        inv = np.float32(2.0 ** -k)
    else:
        s = np.float32(a) / np.float32(448.0)
        inv = np.float32(448.0) / np.float32(a)
    y = (x * inv).astype(np.float32)
    finite = [c for c in range(256) if not np.isnan(table[c])]
    vals = np.array([table[c] for c in finite])
    codes = np.empty(y.size, np.uint8)
    for i, v in enumerate(y.astype(np.float64)):
        mag = min(abs(v), 448.0)
        best = None
        for c, cv in zip(finite, vals):
            if np.signbit(cv) != np.signbit(v):
                continue
            d = abs(abs(cv) - mag)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        codes[i] = best[1]
    return codes, s


def check_quant_bruteforce(orc, seed=7, groups=6):
    """Small random groups (normal draws with outliers, subnormals, zeros and
    ties mixed in) match the brute-force group quantiser exactly."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    for pow2 in (0, 1):
        for gi in range(groups):
            f = rng.standard_normal(128).astype(np.float32) * np.float32(10.0 ** rng.integers(-6, 4))
            f[rng.random(128) < 0.05] *= 100
            f[:3] = [0.0, -0.0, 2.0 ** -130]
            bits = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: still valid bf16
            want, ws = brute_group(bits, pow2, table)
            q, s = orc.quant_tile(bits.reshape(1, 128), 0, pow2)
            np.testing.assert_array_equal(q[0], want, err_msg=f"pow2={pow2} group {gi}")
            assert s[0, 0] == ws


def check_amax_maps_to_448(orc, seed=11):
    """FP32 mode: the group's amax element encodes to +-448 and no code
    exceeds 448 in magnitude (the max absolute value is aligned with the
    largest FP8 value)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    f = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-30, 30, (64, 1))).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quant_tile(bits, 0, 0)
    x = bf16_f32(bits).reshape(64, 4, 128)
    qq = q.reshape(64, 4, 128)
    idx = np.argmax(np.abs(x), axis=2)
    top = np.take_along_axis(qq, idx[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.all(np.abs(table[q]) <= 448)


def check_pow2_exact(orc, seed=13):
    """POW2 mode: the scale is an exact power of two with 224*s < amax <=
    448*s, and values built as (E4M3 value) * 2^k with an element at the top
    binade come back as the same codes with s = 2^k."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    for k in (-20, -7, 0, 5, 30):
        codes = rng.choice(finite, size=(4, 128))
        codes[:, 0] = 0x7C  # 384: amax in (224, 448] so the scale is 2^k
        vals = (table[codes] * 2.0 ** k).astype(np.float32)
        bits = f32_bf16_exact(vals)
        q, s = orc.quant_tile(bits, 0, 1)
        np.testing.assert_array_equal(q, codes)
        assert np.all(s == np.float32(2.0 ** k))
    f = (rng.standard_normal((32, 256)) * 10.0 ** rng.uniform(-20, 20, (32, 1))).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quant_tile(bits, 0, 1)
    amax = np.abs(bf16_f32(bits)).reshape(32, 2, 128).max(axis=2).T
    m, e = np.frexp(s)
    assert np.all(m == 0.5)
    assert np.all(amax <= 448.0 * s) and np.all(amax > 224.0 * s.astype(np.float64))


def check_error_bound(orc, seed=17):
    """|x - dec(q)*s| is within half an E4M3 spacing of the scaled value
    (plus one fp32 rounding of the scaling in FP32 mode)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    f = (rng.standard_normal((16, 1024)) * 3).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    x = bf16_f32(bits).astype(np.float64).reshape(16, 8, 128)
    for pow2 in (0, 1):
        q, s = orc.quant_tile(bits, 0, pow2)
        y = table[q].reshape(16, 8, 128) * s.T[:, :, None].astype(np.float64)
        scaled = np.abs(x) / s.T[:, :, None]
        # spacing of E4M3 at the scaled magnitude: 2^(e-3) for normals,
        # 2^-9 in the subnormal range
        e = np.floor(np.log2(np.maximum(scaled, 2.0 ** -6)))
        half = 0.5 * 2.0 ** (e - 3)
        slack = 0 if pow2 else 2.0 ** -22 * scaled
        assert np.all(np.abs(x / s.T[:, :, None] - y / s.T[:, :, None]) <= half + slack + 1e-30)


def check_transpose_symmetry(orc, seed=19):
    """quant_block(W^T) gives the transposed codes and scales of
    quant_block(W); the transposed copy equals q^T."""
    rng = np.random.default_rng(seed)
    f = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2 in (0, 1):
        q, s, qt = orc.quant_block(bits, pow2, transpose=True)
        q2, s2, _ = orc.quant_block(np.ascontiguousarray(bits.T), pow2)
        np.testing.assert_array_equal(qt, q.T)
        np.testing.assert_array_equal(q2, q.T)
        np.testing.assert_array_equal(s2, s.T)


def check_orientation(orc, seed=23):
    """quant_tile(X, col) equals quant_tile(X^T, row): the 128x1 tiles of the
    backward pass are the 1x128 tiles of the transpose."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((256, 200)).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2 in (0, 1):
        qc, sc = orc.quant_tile(bits, 1, pow2)
        qr, sr = orc.quant_tile(np.ascontiguousarray(bits.T), 0, pow2)
        np.testing.assert_array_equal(qc, qr)
        np.testing.assert_array_equal(sc, sr)


def check_block_vs_rows(orc, seed=29):
    """A 128x128 block whose every row has the same amax quantises exactly
    like those rows in 1x128 groups."""
    rng = np.random.default_rng(seed)
    f = rng.uniform(-1, 1, (128, 256)).astype(np.float32)
    f[:, 5] = 3.0
    f[:, 130] = -3.0
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2 in (0, 1):
        qb, sb, _ = orc.quant_block(bits, pow2)
        qr, sr = orc.quant_tile(bits, 0, pow2)
        np.testing.assert_array_equal(qb, qr)
        assert np.all(sr == sb[0][:, None])


# ---- 128x1 groups per expert ---------------------------------------------------------

def check_grouped_col_aligned(orc, seed=59):
    """When every expert's token count is a multiple of 128 there is no
    padding, and the per-expert grouping equals quant_tile(axis 1) of each
    expert's rows, concatenated along the token axis."""
    rng = np.random.default_rng(seed)
    counts = [128, 0, 256, 128]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    f = (rng.standard_normal((int(offsets[-1]), 192)) * 10.0 ** rng.uniform(-3, 3, (int(offsets[-1]), 1))).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2 in (0, 1):
        q, s = orc.quant_tile_grouped_col(bits, offsets, pow2)
        assert q.shape == (192, 512) and s.shape == (4, 192)
        for e in range(len(counts)):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 == r0:
                continue
            qe, se = orc.quant_tile(np.ascontiguousarray(bits[r0:r1]), 1, pow2)
            np.testing.assert_array_equal(q[:, r0:r1], qe)
            np.testing.assert_array_equal(s[r0 // 128:r1 // 128], se)


def check_grouped_col_partial(orc, seed=61):
    """Ragged experts (0, 1, 130, 0, 257, 40 tokens): every group, the
    partial last ones included, matches the brute-force group quantiser on
    exactly that expert's tokens, the padding holds zero codes, and each
    expert starts on a 128-token boundary of the padded axis."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    counts = [0, 1, 130, 0, 257, 40]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    f = (rng.standard_normal((int(offsets[-1]), 16)) * 3).astype(np.float32)
    f[rng.random(f.shape) < 0.02] *= 100
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2 in (0, 1):
        q, s = orc.quant_tile_grouped_col(bits, offsets, pow2)
        assert q.shape == (16, 7 * 128) and s.shape == (7, 16)
        start = 0
        for e, n in enumerate(counts):
            for j in range((n + 127) // 128):
                length = min(128, n - 128 * j)
                rows = int(offsets[e]) + 128 * j + np.arange(length)
                for c in (0, 5, 15):
                    want, ws = brute_group(bits[rows, c], pow2, table)
                    got = q[c, start + 128 * j:start + 128 * j + 128]
                    np.testing.assert_array_equal(got[:length], want, err_msg=f"pow2={pow2} e={e} j={j} c={c}")
                    assert np.all(got[length:] == 0)
                    assert s[start // 128 + j, c] == ws
            start += (n + 127) // 128 * 128


# ---- backward re-tiling ------------------------------------------------------------

def check_requant_bruteforce(orc, seed=47):
    """Re-tiling 1x128 codes into 128x1 groups: sampled output groups match
    the brute-force group quantiser applied to the fp32 dequantised column
    (numpy's IEEE fp32 product of the decoded code and its row scale)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    f = (rng.standard_normal((256, 256)) * 10.0 ** rng.uniform(-3, 3, (256, 1))).astype(np.float32)
    f[rng.random(f.shape) < 0.01] *= 100
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    for pow2_in in (0, 1):
        q, s = orc.quant_tile(bits, 0, pow2_in)
        for pow2 in (0, 1):
            qt, st = orc.requant_col(q, s, pow2)
            assert qt.shape == (256, 256) and st.shape == (2, 256)
            for c in (0, 77, 128, 255):
                for g in (0, 1):
                    rows = np.arange(g * 128, g * 128 + 128)
                    xhat = table[q[rows, c]].astype(np.float32) * s[c // 128, rows]
                    want, ws = brute_group_f32(xhat, pow2, table)
                    np.testing.assert_array_equal(qt[c, g * 128:(g + 1) * 128], want,
                                                  err_msg=f"in={pow2_in} out={pow2} col {c} group {g}")
                    assert st[g, c] == ws


def check_requant_exact_dequant(orc, seed=53):
    """With power-of-two row scales the dequantised values (4 significant
    bits) are exact bf16 numbers, so re-tiling must equal quantising that
    exact matrix directly in 128x1 groups."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    f = (rng.standard_normal((384, 256)) * 10.0 ** rng.uniform(-2, 2, (384, 1))).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quant_tile(bits, 0, 1)
    xhat = table[q] * np.repeat(s.T, 128, axis=1).astype(np.float64)
    xbits = f32_bf16_exact(xhat.astype(np.float32))
    for pow2 in (0, 1):
        qt, st = orc.requant_col(q, s, pow2)
        qd, sd = orc.quant_tile(xbits, 1, pow2)
        np.testing.assert_array_equal(qt, qd)
        np.testing.assert_array_equal(st, sd)


def check_requant_fp32_dequant(orc):
    """Worked case for the reading that the dequantised element is the fp32
    product fl32(dec(q) * s).  Column 0 holds 448 (code 0x7E, row scale 1)
    and 1.25 (code 0x3A) with the row scale fl32(0.85) = 0.85000002384...:
    the exact product 1.0625000298... lies just above 1.0625, the midpoint of
    E4M3 1.0 (0x38) and 1.125 (0x39), but rounds to 1.0625 in fp32.  The
    group amax is 448, so the new scale is 1 and the element's code is the
    tie, broken to the even code 0x38 (rounding the exact product would give
    0x39)."""
    s1 = np.float32(0.85)
    assert fractions.Fraction(5, 4) * fractions.Fraction(float(s1)) > fractions.Fraction(17, 16)
    assert np.float32(1.25) * s1 == np.float32(1.0625)
    q = np.zeros((128, 128), np.uint8)
    s = np.ones((1, 128), np.float32)
    q[0, 0], q[1, 0] = 0x7E, 0x3A
    s[0, 1] = s1
    for pow2 in (0, 1):
        qt, st = orc.requant_col(q, s, pow2)
        assert st[0, 0] == np.float32(1.0)
        assert qt[0, 0] == 0x7E and qt[0, 1] == 0x38, (pow2, hex(qt[0, 1]))
        assert np.all(qt[0, 2:] == 0)


# ---- GEMM -------------------------------------------------------------------------

def _random_codes(rng, shape, table):
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    return rng.choice(finite, size=shape)


def check_gemm_bruteforce(orc, seed=31):
    """Tiny GEMMs against an independent fp64 dequantise-then-multiply
    (numpy, per group), for both B-scale kinds; relative error <= 1e-12."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    M, N, K = 7, 130, 384
    a = _random_codes(rng, (M, K), table)
    b = _random_codes(rng, (N, K), table)
    sa = rng.uniform(0.1, 4, (K // 128, M)).astype(np.float32)
    A = table[a]
    B = table[b]
    # block kind: SB(n, g) = sbk[n // 128, g]
    sbk = rng.uniform(0.1, 4, ((N + 127) // 128, K // 128)).astype(np.float32)
    want = np.zeros((M, N))
    for g in range(K // 128):
        ks = slice(128 * g, 128 * g + 128)
        sbn = sbk[np.arange(N) // 128, g].astype(np.float64)
        want += (A[:, ks] * sa[g][:, None]) @ (B[:, ks] * sbn[:, None]).T
    got = orc.gemm(a, sa, b, sbk, 0, sbk.shape[1], 1)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # the same block scales addressed through swapped strides (Dgrad layout)
    sbt = np.ascontiguousarray(sbk.T)
    got2 = orc.gemm(a, sa, b, sbt, 0, 1, sbt.shape[1])
    np.testing.assert_array_equal(got, got2)
    # tile kind: SB(n, g) = sbc[g, n]
    sbc = rng.uniform(0.1, 4, (K // 128, N)).astype(np.float32)
    want = np.zeros((M, N))
    for g in range(K // 128):
        ks = slice(128 * g, 128 * g + 128)
        want += (A[:, ks] * sa[g][:, None]) @ (B[:, ks] * sbc[g][:, None].astype(np.float64)).T
    got = orc.gemm(a, sa, b, sbc, 1, N, 0)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def check_gemm_identity(orc, seed=37):
    """A = identity (code 0x38 = 1.0 on the diagonal, scale 1) gives exactly
    the dequantised B^T, power-of-two scales included."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    K = N = 256
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = 0x38
    sa = np.ones((K // 128, K), np.float32)
    b = _random_codes(rng, (N, K), table)
    sbk = (2.0 ** rng.integers(-20, 20, (N // 128, K // 128))).astype(np.float32)
    got = orc.gemm(a, sa, b, sbk, 0, sbk.shape[1], 1)
    want = (table[b] * sbk[np.arange(N)[:, None] // 128, np.arange(K)[None, :] // 128]).T
    np.testing.assert_array_equal(got, want)


def check_gemm_integers(orc, seed=41):
    """Codes of small integers with unit scales: the result is the integer
    matrix product (numpy int64)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    ints = {int(v): c for c, v in enumerate(table) if not np.isnan(v) and v == int(v) and abs(v) <= 8 and c != 0x80}
    keys = np.array(sorted(ints))
    M, N, K = 33, 65, 512
    ia = rng.choice(keys, (M, K))
    ib = rng.choice(keys, (N, K))
    a = np.vectorize(ints.get)(ia).astype(np.uint8)
    b = np.vectorize(ints.get)(ib).astype(np.uint8)
    got = orc.gemm(a, np.ones((K // 128, M), np.float32), b,
                   np.ones((1, K // 128), np.float32), 0, 0, 1)
    np.testing.assert_array_equal(got, (ia.astype(np.int64) @ ib.T.astype(np.int64)).astype(np.float64))


def check_gemm_entries_and_grouped(orc, seed=43):
    """gemm_entries agrees with gemm; the grouped GEMM equals one dense GEMM
    per expert (empty experts included)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    M, N, K = 40, 256, 256
    a = _random_codes(rng, (M, K), table)
    b = _random_codes(rng, (N, K), table)
    sa = rng.uniform(0.5, 2, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    full = orc.gemm(a, sa, b, sb, 0, K // 128, 1)
    mi = rng.integers(0, M, 50)
    ni = rng.integers(0, N, 50)
    np.testing.assert_array_equal(orc.gemm_entries(a, sa, b, sb, 0, K // 128, 1, mi, ni), full[mi, ni])
    G = 3
    offsets = np.array([0, 17, 17, 40], np.int32)
    bg = _random_codes(rng, (G, N, K), table)
    sbg = rng.uniform(0.5, 2, (G, N // 128, K // 128)).astype(np.float32)
    got = orc.grouped_gemm(offsets, a, sa, bg, sbg)
    for e in range(G):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        want = orc.gemm(a[r0:r1], sa[:, r0:r1], bg[e], sbg[e], 0, K // 128, 1)
        np.testing.assert_array_equal(got[r0:r1], want)
    np.testing.assert_array_equal(orc.grouped_gemm_entries(offsets, a, sa, bg, sbg, mi, ni), got[mi, ni])


def check_scale_edges(orc):
    """The amax floor and the limits of both scale modes."""
    fl = orc.amax_floor()
    assert fl == np.float32(448.0 * 2.0 ** -126)
    for pow2 in (0, 1):
        s, inv = orc.group_scale(0.0, pow2)
        assert s == np.float32(2.0 ** -126) and inv == np.float32(2.0 ** 126)
    biggest = np.float32(bf16_f32(np.uint16(0x7F7F)))
    s, inv = orc.group_scale(biggest, 1)
    assert s == np.float32(2.0 ** 120) and inv == np.float32(2.0 ** -120)
    s, inv = orc.group_scale(biggest, 0)
    assert np.isfinite(s) and inv > 0
    assert orc.group_scale(448.0, 1) == (np.float32(1.0), np.float32(1.0))
    assert orc.group_scale(448.5, 1)[0] == np.float32(2.0)
    assert orc.group_scale(224.0, 1)[0] == np.float32(0.5)
    assert orc.group_scale(224.5, 1)[0] == np.float32(1.0)


# ---- limited-precision accumulation model -------------------------------------------

def load_limited():
    rows = []
    with open(os.path.join(GOLDEN, "limited_accumulation.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, K, first, rest, bits, chunk, interval, want = line.split()
            rows.append((name, int(K), int(first, 16), int(rest, 16), int(bits), int(chunk), int(interval),
                         float(want)))
    return rows


def check_limited_worked(orc):
    """The model of limited accumulation on the hand-worked cases of
    tests/golden/limited_accumulation.txt (swamping of small products by a
    large one, cutting toward zero, exact chunks, promotion intervals)."""
    rows = load_limited()
    assert len(rows) >= 9
    for name, K, first, rest, bits, chunk, interval, want in rows:
        a = np.full((1, K), rest, np.uint8)
        a[0, 0] = first
        b = np.full((1, K), 0x38, np.uint8)
        sa = np.ones((K // 128, 1), np.float32)
        sb = np.ones((1, K // 128), np.float32)
        got = orc.gemm_limited(a, sa, b, sb, 0, K // 128, 1, bits, chunk, interval)
        assert got[0, 0] == want, (name, got[0, 0], want)


def check_limited_reduces_to_exact(orc, seed=67):
    """With 53 bits the model is the plain sum: promoted every 128 elements
    it equals the oracle's GEMM bit for bit (each group partial is exact in
    fp64 and is scaled and added in the same order), and never promoted with
    unit scales it equals the exact integer-unit sum too; fewer bits never
    beat the exact result on these inputs by construction of the cut
    (|limited| <= |exact| for a sum of same-sign products)."""
    rng = np.random.default_rng(seed)
    table = orc.decode_table()
    M, N, K = 5, 140, 512
    a = _random_codes(rng, (M, K), table)
    b = _random_codes(rng, (N, K), table)
    sa = rng.uniform(0.1, 4, (K // 128, M)).astype(np.float32)
    sbk = rng.uniform(0.1, 4, ((N + 127) // 128, K // 128)).astype(np.float32)
    exact = orc.gemm(a, sa, b, sbk, 0, sbk.shape[1], 1)
    np.testing.assert_array_equal(orc.gemm_limited(a, sa, b, sbk, 0, sbk.shape[1], 1, 53, 1, 128), exact)
    sbc = rng.uniform(0.1, 4, (K // 128, N)).astype(np.float32)
    np.testing.assert_array_equal(orc.gemm_limited(a, sa, b, sbc, 1, N, 0, 53, 4, 128),
                                  orc.gemm(a, sa, b, sbc, 1, N, 0))
    ones_a = np.ones((K // 128, M), np.float32)
    ones_b = np.ones((2, K // 128), np.float32)
    np.testing.assert_array_equal(orc.gemm_limited(a, ones_a, b, ones_b, 0, K // 128, 1, 53, 1, 0),
                                  orc.gemm(a, ones_a, b, ones_b, 0, K // 128, 1))
    pos_a, pos_b = a & np.uint8(0x7F), b & np.uint8(0x7F)
    lim = orc.gemm_limited(pos_a, sa, pos_b, sbk, 0, sbk.shape[1], 1, 10, 1, 0)
    full = orc.gemm(pos_a, sa, pos_b, sbk, 0, sbk.shape[1], 1)
    assert np.all(lim <= full) and np.all(lim >= full * (1 - 2.0 ** -9 * K))


ALL_CHECKS = [
    check_decode_table, check_round_trip, check_anchors, check_worked_examples,
    check_quant_bruteforce, check_amax_maps_to_448, check_pow2_exact,
    check_error_bound, check_transpose_symmetry, check_orientation,
    check_block_vs_rows, check_gemm_bruteforce, check_gemm_identity,
    check_gemm_integers, check_gemm_entries_and_grouped, check_scale_edges,
    check_requant_bruteforce, check_requant_exact_dequant, check_requant_fp32_dequant,
    check_grouped_col_aligned, check_grouped_col_partial,
    check_limited_worked, check_limited_reduces_to_exact,
]

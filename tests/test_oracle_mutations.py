"""Mutation tests: plant one plausible mistake in a copy of oracle.c, build
it on the CPU, and require that the pins of pinlib reject it.  This shows the
pins are strong enough to catch a dropped term, a wrong rounding, a wrong
index or a transposed operand in the oracle.  CPU only."""
import os
import tempfile

import pytest

import oracle
from oracle import build as obuild
import pinlib

SRC = open(obuild.SRC).read()

MUTATIONS = {
    "ties_away_from_zero": (
        "return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;",
        "return f + 1.0;"),
    "saturate_too_late": (
        "if (a >= 448.0)\n        return (uint8_t)(sign | 0x7E);",
        "if (a >= 480.0)\n        return (uint8_t)(sign | 0x7E);"),
    "subnormal_step_wrong": (
        "double m = round_half_even(a * 512.0);",
        "double m = round_half_even(a * 256.0);"),
    "sign_dropped": (
        "uint8_t sign = signbit(v) ? 0x80 : 0x00;",
        "uint8_t sign = v < 0.0f ? 0x80 : 0x00;"),
    "pow2_rounded_down": (
        "    *s = (float)ldexp(1.0, k);\n    *inv = (float)ldexp(1.0, -k);",
        "    k -= 1;\n    *s = (float)ldexp(1.0, k);\n    *inv = (float)ldexp(1.0, -k);"),
    "fnuz_max_240": (
        "*s = a / 448.0f;\n        *inv = 448.0f / a;",
        "*s = a / 240.0f;\n        *inv = 240.0f / a;"),
    "no_amax_floor": (
        "float a = amax > floor_a ? amax : floor_a;",
        "float a = amax > 0.0f ? amax : 1.0f;"),
    "col_groups_along_rows": (
        "quantise_group(x + (g * 128) * ldx + c, ldx, 128, pow2,",
        "quantise_group(x + (g * 128) * ldx + c, 1, 128, pow2,"),
    "block_amax_first_row_only": (
        "            for (int64_t r = 0; r < nr; r++)\n                for (int64_t c = 0; c < 128; c++) {\n                    float v = fabsf(",
        "            for (int64_t r = 0; r < 1; r++)\n                for (int64_t c = 0; c < 128; c++) {\n                    float v = fabsf("),
    "transposed_block_copy": (
        "qt[(c0 + c) * ldqt + r0 + r] = code;",
        "qt[(c0 + c) * ldqt + r0 + r] = q[(r0 + r) * ldq + c0 + (127 - c)];"),
    "group_partial_short": (
        "for (int64_t k = g * 128; k < g * 128 + 128; k++)",
        "for (int64_t k = g * 128; k < g * 128 + 127; k++)"),
    "b_scale_dropped": (
        "double scale = (double)sa[g * ldsa + m] * sb_at(sb, kind, s0, s1, n, g);",
        "double scale = (double)sa[g * ldsa + m];"),
    "b_scale_strides_swapped": (
        "return (double)sb[(n / 128) * s0 + g * s1];",
        "return (double)sb[(n / 128) * s1 + g * s0];"),
    "a_scale_wrong_group": (
        "double scale = (double)sa[g * ldsa + m] * sb_at",
        "double scale = (double)sa[((g + 1) % (K / 128)) * ldsa + m] * sb_at"),
    "tile_scale_per_block": (
        "return (double)sb[g * s0 + n];",
        "return (double)sb[g * s0 + (n / 128) * 128];"),
    "requant_dequant_to_bf16": (
        "x[i] = d * s[(c / 128) * lds + r];                /* fp32 */",
        "{ float t = d * s[(c / 128) * lds + r]; uint32_t u; memcpy(&u, &t, 4);\n"
        "  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u; memcpy(&x[i], &u, 4); }"),
    "requant_scale_wrong_row": (
        "x[i] = d * s[(c / 128) * lds + r];",
        "x[i] = d * s[(c / 128) * lds + (r ^ 1)];"),
    "requant_amax_of_codes": (
        "                if (fabsf(x[i]) > amax)\n                    amax = fabsf(x[i]);\n            }\n            /* quantise again",
        "                if (fabsf(d) > amax)\n                    amax = fabsf(d);\n            }\n            /* quantise again"),
    "requant_not_transposed": (
        "qt[c * ldqt + g * 128 + i] = orc_e4m3_encode(x[i] * inv);",
        "qt[(g * 128 + i) * cols + c] = orc_e4m3_encode(x[i] * inv);"),
    "grouped_col_padding_not_zero": (
        "                    out[i] = 0; /* padding */",
        "                    out[i] = 0x7E; /* padding */"),
    "grouped_col_scale_slot_first_group": (
        "s[(start / 128 + j) * lds + c] =",
        "s[(start / 128) * lds + c] ="),
    "grouped_col_unpadded_start": (
        "        start += ng * 128;",
        "        start += n;"),
    "limited_cut_to_nearest": (
        "double t = floor(ldexp(fr, bits)); /* the top `bits` bits as an integer */",
        "double t = floor(ldexp(fr, bits) + 0.5);"),
    "limited_partial_not_restarted": (
        "double part = limited_sum(0.0, prod, interval, chunk, bits);",
        "double part = limited_sum(out, prod, interval, chunk, bits) - out;"),
    "limited_chunk_ignored": (
        "        for (int64_t j = i; j < i + chunk && j < n; j++)",
        "        for (int64_t j = i; j < i + 1 && j < n; j++)"),
    "b_reversed_within_group": (
        "p += (int64_t)dec_units[arow[k]] * (int64_t)dec_units[brow[k]];",
        "p += (int64_t)dec_units[arow[k]] * (int64_t)dec_units[brow[g * 128 + 127 - (k - g * 128)]];"),
}


def _run_pins(orc):
    """Names of the pins that reject this oracle."""
    failed = []
    for check in pinlib.ALL_CHECKS:
        try:
            check(orc)
        except Exception:  # an error code from the oracle also counts
            failed.append(check.__name__)
    try:
        pinlib.check_codec_exhaustive(orc, stride=4099)
    except AssertionError:
        failed.append("check_codec_exhaustive(sampled)")
    return failed


def test_unmutated_oracle_passes(orc):
    assert _run_pins(orc) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation {name} no longer applies"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "oracle.c")
        with open(src, "w") as f:
            f.write(SRC.replace(old, new))
        # the header sits next to the real source
        lib = obuild.build(src=src, out=os.path.join(d, "liboracle_mut.so"),
                           extra=("-I", os.path.dirname(obuild.SRC)))
        failed = _run_pins(oracle.Oracle(lib))
    assert failed, f"no pin rejects the planted mistake {name}"

"""CPU-only pins of the oracle (no GPU).  See ``oracle_checks.py`` for what each
check compares the oracle against."""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_checks as oc

CHECKS = oc.ALL_CHECKS


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check()


# Plausible mistakes, planted in a copy of the oracle's source.  Each mutant is
# (description, text in fp4_oracle.c, replacement).  Every one of them must make
# at least one pin fail; otherwise the pins would not be pinning that part.
MUTANTS = [
    ("mx exponent off by one", "int e = (E - 1) - 2;", "int e = (E - 1) - 1;"),
    ("e2m1 ties away from even", "if (d < bestd || (d == bestd && (c & 1) == 0)) {\n            best = c;\n            bestd = d;\n        }\n    }\n    return (neg << 3) | best;",
     "if (d < bestd || (d == bestd && (c & 1) == 1)) {\n            best = c;\n            bestd = d;\n        }\n    }\n    return (neg << 3) | best;"),
    ("e2m1 subnormal step", "mag = 0.5 * man;", "mag = 1.0 * man;"),
    ("e2m1 exponent bias", "mag = ldexp(1.0 + 0.5 * man, exp_field - 1);", "mag = ldexp(1.0 + 0.5 * man, exp_field);"),
    ("e4m3 subnormal step", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("e4m3 bias", "mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    ("e4m3 ties", "if (d < bestd || (d == bestd && (c & 1) == 0)) {\n            best = c;\n            bestd = d;\n        }\n    }\n    return best;",
     "if (d < bestd) {\n            best = c;\n            bestd = d;\n        }\n    }\n    return best;"),
    ("nv tensor scale forgets the 6", "tsv = gamax / 2688.0f;", "tsv = gamax / 448.0f;"),
    ("nv block scale order", "float t = (amax / 6.0f) / tsv;", "float t = amax / (6.0f * tsv) * 1.0001f;"),
    ("nv dequant drops tensor scale", "dst[r * cols + k] = inner * ts;", "dst[r * cols + k] = inner;"),
    ("nibble order swapped", "if ((k & 1) == 0)\n        row_codes[k >> 1]", "if ((k & 1) == 1)\n        row_codes[k >> 1]"),
    ("hadamard sign pattern", "(unsigned)(i & j)", "(unsigned)(i | j)"),
    ("hadamard normalisation", "float v = (float)(s / root);", "float v = (float)(s / n);"),
    ("block amax without abs", "float a = fabsf(v[i]);", "float a = v[i];"),
    ("mx clamp", "if (e < -127)\n        e = -127;", "if (e < -126)\n        e = -126;"),
    ("gemm drops a sign", "s += av * bv;", "s += av * fabs(bv);"),
    ("gemm forgets tensor scales", "s *= g;", "s *= 1.0;"),
    ("gemm transposed scale index", "bsv = ora_e8m0_decode(bs[b]);", "bsv = ora_e8m0_decode(as[b]);"),
    ("error sums drop a term", "se += (a - b) * (a - b);", "se += (a - b) * (a - b) * 0.5;"),
    ("w4a16 drops the weight tensor scale", "s *= (double)b_ts;", "s *= 1.0;"),
    ("w4a16 loses the activation sign", "s += (double)ar[k] * bv;", "s += fabs((double)ar[k]) * bv;"),
    ("w4a16 scale of the next block", "double bsv = fmt_mx(fmt) ? ora_e8m0_decode(bs[b]) : ora_e4m3_decode(bs[b]);",
     "double bsv = fmt_mx(fmt) ? ora_e8m0_decode(bs[(b + 1) % nb]) : ora_e4m3_decode(bs[(b + 1) % nb]);"),
    ("mse window skips e0+1", "cands[nc++] = sc + 1;", "cands[nc++] = sc + 2;"),
    ("mse nv window loses c0-1", "nv_window[9] = {0, 1, -1, 2,", "nv_window[9] = {0, 1, 1, 2,"),
    ("mse ties go to later candidates", "if (e < best) {", "if (e <= best) {"),
    ("mse error not squared", "acc = fmaf(d, d, acc);", "acc = acc + fabsf(d);"),
    ("mse scores a candidate with the old codes", "float e = block_sse(fmt, yb, G, c, tsv, cand_code);",
     "float e = block_sse(fmt, yb, G, c, tsv, code);"),
    ("four over six maps to 3", "nv_scale_code(amax, 4.0f, tsv)", "nv_scale_code(amax, 3.0f, tsv)"),
    ("int4 ties away from even", "if (d < bestd || (d == bestd && (m & 1) == 0)) {",
     "if (d < bestd || (d == bestd && (m & 1) == 1)) {"),
    ("int4 saturates at 8 (two's-complement range)",
     "if (a > 7.0)\n        a = 7.0;\n    int best = 0;\n    double bestd = INFINITY;\n    for (int m = 0; m <= 7; ++m) {",
     "if (a > 8.0)\n        a = 8.0;\n    int best = 0;\n    double bestd = INFINITY;\n    for (int m = 0; m <= 8; ++m) {"),
    ("int4 decode without sign extension", "return c >= 8 ? (double)(c - 16) : (double)c;",
     "return c >= 8 ? (double)(8 - c) : (double)c;"),
    ("nvint4 tensor scale uses the FP4 maximum", "tsv = gamax / 3136.0f;", "tsv = gamax / 2688.0f;"),
    ("nvint4 block scale divides by 6", "float t = (amax / 7.0f) / tsv;", "float t = (amax / 6.0f) / tsv;"),
    ("philox multiplier", "(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F55u * c0"),
    ("philox key schedule", "k1 += 0xBB67AE85u;", "k1 += 0xBB67AE86u;"),
    ("stochastic rounding ties up", "if (u < p)\n            mag = lo + 1;", "if (u <= p)\n            mag = lo + 1;"),
    ("stochastic rounding reuses one word", "return (double)(out[e & 3] >> 8) * 0x1p-24;",
     "return (double)(out[0] >> 8) * 0x1p-24;"),
    ("rotation signs indexed by output", "xi *= sign_of(signs, i);", "xi *= sign_of(signs, j);"),
    ("rotation sign bit within a word", "return ((signs[i >> 5] >> (i & 31)) & 1u) ? -1.0 : 1.0;",
     "return ((signs[i >> 5] >> (i & 15)) & 1u) ? -1.0 : 1.0;"),
    ("two-dimensional tile of 8 rows", "long r0 = r - r % q->block_rows;", "long r0 = r - r % 8;"),
    ("int4 formats decode as E2M1", "return fmt_int(fmt) ? ora_int4_decode(code) : ora_e2m1_decode(code);",
     "return ora_e2m1_decode(code);"),
    ("tiles ordered down the panels first", "long start = (panel * tiles_per_panel + tile) * 8192;",
     "long start = (tile * (rows / 128) + panel) * 8192;"),
    ("tile stored column-major", "dst[start + (r % 128) * 64 + (b % 64)]", "dst[start + (b % 64) * 128 + (r % 128)]"),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant):
    name, old, new = mutant
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutant anchor must be unique: " + name
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", so, c, "-lm"])
        oracle.use_library(so)
        failed = []
        try:
            for chk in CHECKS:
                try:
                    chk()
                except AssertionError:
                    failed.append(chk.__name__)
                    break
        finally:
            oracle.use_library(None)
    assert failed, "no pin caught the planted mistake: " + name

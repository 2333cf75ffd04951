"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``check_*`` function raises AssertionError on a mismatch.  They are run by
``test_oracle_pins.py`` against the real oracle, and by the mutation test
against deliberately broken copies of it (every planted mistake must trip at
least one check).  None of these checks re-types the oracle's own algorithm:
each compares it with a printed value, a closed form, a library routine, an
invariant, or a brute-force search.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.linalg

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


FMT = _golden("format_definitions.json")
GRID = np.array(FMT["e2m1_positive_magnitudes"])          # index = magnitude code


# ---------------------------------------------------------------- E2M1 codec
def check_e2m1_value_set():
    """Format definitions: the 16 codes decode to {0, +-0.5, ..., +-6}; bit 3 is
    the sign; exponent field bias 1 puts 1.0 at 0b0010, 2.0 at 0b0100, 4.0 at
    0b0110 and 6.0 (=1.5 * 4) at 0b0111."""
    vals = np.array([oracle.e2m1_decode(c) for c in range(16)])
    assert np.array_equal(vals[:8], GRID), vals
    assert np.array_equal(vals[8:], -GRID), vals
    assert oracle.e2m1_decode(0b0010) == 1.0 and oracle.e2m1_decode(0b0100) == 2.0
    assert oracle.e2m1_decode(0b0110) == 4.0 and oracle.e2m1_decode(0b0111) == 6.0
    assert oracle.e2m1_decode(0b0001) == 0.5          # subnormal 0.1b x 2^0
    # code 8 is negative zero
    assert oracle.e2m1_decode(8) == 0.0 and np.signbit(oracle.e2m1_decode(8))


def check_e2m1_midpoints():
    """Round-to-nearest-even onto the grid (training recipe: RNE for weights and
    activations).  Midpoints between neighbours resolve to the even code
    (mantissa bit 0): 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4."""
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for m, v in expect.items():
        c = oracle.e2m1_encode(m)
        assert oracle.e2m1_decode(c) == v, (m, c)
        assert oracle.e2m1_decode(oracle.e2m1_encode(-m)) == -v
        up = np.nextafter(np.float32(m), np.float32(10))
        dn = np.nextafter(np.float32(m), np.float32(0))
        i = int(np.searchsorted(GRID, m))                   # GRID[i-1] < m < GRID[i]
        assert oracle.e2m1_decode(oracle.e2m1_encode(up)) == GRID[i], (m, "up")
        assert oracle.e2m1_decode(oracle.e2m1_encode(dn)) == GRID[i - 1], (m, "down")


def _float_rne_e2m1(q: np.ndarray) -> np.ndarray:
    """E2M1 rounding written as generic floating-point rounding: find the binade
    of |q| (minimum exponent 1 - bias = 0), the spacing there is 2^(E-1) (one
    mantissa bit), round to a multiple of it with ties to even (np.rint), then
    saturate at the largest finite value 6."""
    a = np.abs(q.astype(np.float64))
    a = np.minimum(a, 6.0)
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    E = np.maximum(E, 0.0)
    step = np.exp2(E - 1.0)
    r = np.rint(a / step) * step
    r = np.minimum(r, 6.0)
    mag = np.searchsorted(GRID, r)
    assert np.array_equal(GRID[mag], r)
    return (np.signbit(q).astype(np.uint8) << 3) | mag.astype(np.uint8)


def _e2m1_probe_values() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)                       # every bf16 pattern
    f = f[np.isfinite(f)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 8.0], np.float32)
    more = []
    for m in mids:
        v = np.float32(m)
        lo = hi = v
        for _ in range(4):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(100))
            more += [lo, hi]
    rnd = workloads.rng(11, 11).uniform(-8, 8, 20000).astype(np.float32)
    return np.concatenate([f, mids, -mids, np.array(more, np.float32),
                           -np.array(more, np.float32), rnd]).astype(np.float32)


def check_e2m1_exhaustive_vs_float_rounding():
    """All bf16 bit patterns plus a dense neighbourhood of every midpoint: the
    oracle's nearest-grid-point encoder equals generic binade-wise RNE with
    saturation at 6."""
    q = _e2m1_probe_values()
    got = oracle.e2m1_encode_array(q)
    ref = _float_rne_e2m1(q)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (q[bad[:5]], got[bad[:5]], ref[bad[:5]])


def check_e2m1_saturation_and_sign():
    assert oracle.e2m1_encode(1e30) == 0x7 and oracle.e2m1_encode(-1e30) == 0xF
    assert oracle.e2m1_encode(6.5) == 0x7 and oracle.e2m1_encode(7.99) == 0x7
    assert oracle.e2m1_encode(0.0) == 0x0
    assert oracle.e2m1_encode(-0.1) == 0x8                  # sign of a value rounded to 0
    assert oracle.e2m1_encode(-0.0) == 0x8


# ---------------------------------------------------------------- E4M3 codec
def _e4m3_values_from_definition():
    """Non-negative finite E4M3 values from the definition: 3 mantissa bits,
    minimum normal exponent -6 (subnormal spacing 2^-9), maximum 448."""
    vals = [m * 2.0 ** -9 for m in range(8)]                 # subnormals (and 0)
    for e in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e
            if v <= FMT["e4m3_max"]:
                vals.append(v)
    return np.array(vals)


def check_e4m3_decode():
    vals = _e4m3_values_from_definition()
    assert vals.size == 127
    got = np.array([oracle.e4m3_decode(c) for c in range(127)])
    assert np.array_equal(got, vals), np.nonzero(got != vals)
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6 and oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x80 | 0x38) == -1.0


def _binade_rne_e4m3(t: np.ndarray) -> np.ndarray:
    """E4M3 rounding binade by binade, the way "NVFP4 vs MXFP4: 4-Bit Floating
    Point for LLM Training and Inference (2026)" emulates it in its section
    "Emulating both formats yourself": clip to [0, 448], take the binade
    exponent (floored at -6, the subnormal range), round onto that binade's
    spacing 2^(e-3) with ties to even; returns the value.  A different
    algorithm from the oracle's nearest-value scan, so it pins the oracle's
    E4M3 encoder to the page's definition."""
    x = np.clip(t.astype(np.float64), 0, 448)
    out = np.zeros_like(x)
    m = x > 0
    e = np.maximum(np.floor(np.log2(x[m])), -6)
    step = np.exp2(e - 3)
    out[m] = np.rint(x[m] / step) * step
    return np.minimum(out, 448)


def check_e4m3_encode_exhaustive():
    vals = _e4m3_values_from_definition()
    mids = (vals[1:] + vals[:-1]) / 2
    probe = [vals, mids, np.array([448.0, 460.0, 464.0, 480.0, 1e4, 1e30, np.inf])]
    for arr in (vals, mids):
        f = arr.astype(np.float32)
        lo, hi = f.copy(), f.copy()
        for _ in range(3):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(1e9))
            probe += [lo, hi]
    probe.append(np.exp2(workloads.rng(12, 12).uniform(-14, 10, 50000)))
    t = np.concatenate(probe).astype(np.float32)
    codes = oracle.e4m3_encode_array(t)
    got = np.array([vals[c] for c in codes])
    ref = _binade_rne_e4m3(t)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (t[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # ties go to the even code
    for i in range(1, 127):
        mid = np.float32((vals[i - 1] + vals[i]) / 2)
        if float(mid) == (vals[i - 1] + vals[i]) / 2:
            c = oracle.e4m3_encode(mid)
            assert c in (i - 1, i) and c % 2 == 0, (i, c)
    assert oracle.e4m3_encode(0.0) == 0 and oracle.e4m3_encode(1e30) == 0x7E


def check_tensor_scale_alone():
    """The tensor scale on its own equals the one quantize() computes, the
    worked example's 2.6 / 2688 ("NVFP4 vs MXFP4 ...", "A worked example, by
    hand"), the closed form max|x| / 2688 (or / 3136 for NVINT4) in fp32,
    and over row chunks its maximum is the whole tensor's (so a tensor can be
    scaled chunk by chunk)."""
    ex = np.array([0.1, -0.3, 0.7, 1.1, -0.2, 0.05, 0.9, 2.6] + [0.0] * 8, np.float32)
    assert oracle.tensor_scale(ex, oracle.NVFP4) == np.float32(2.6) / np.float32(2688.0)
    x = workloads.bf16_bits_to_f32(workloads.cfg2_tensor("laplace", 3, rows=96, cols=256))
    for fmt, div in ((oracle.NVFP4, 2688.0), (oracle.NVINT4, 3136.0)):
        assert oracle.tensor_scale(x, fmt) == np.float32(np.abs(x).max()) / np.float32(div)
        for rot in (False, True):
            _, _, ts = oracle.quantize(x, fmt, rotate=rot)
            assert oracle.tensor_scale(x, fmt, rotate=rot) == ts
            parts = [oracle.tensor_scale(x[i:i + 17], fmt, rotate=rot) for i in range(0, 96, 17)]
            assert max(parts) == ts
    for bad in ((x, oracle.MXFP4), (x[:, :250], oracle.NVFP4)):
        try:
            oracle.tensor_scale(*bad)
        except ValueError:
            continue
        raise AssertionError("tensor_scale accepted a bad call")


def check_e8m0():
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(0) == 2.0 ** -127 and oracle.e8m0_decode(254) == 2.0 ** 127
    assert oracle.e8m0_decode(126) == 0.5


# --------------------------------------------------------- worked examples
def check_worked_example_mxfp4():
    g = _golden("vs_worked_example.json")
    x = np.zeros(32, np.float32)
    x[:8] = g["values"]
    codes, scales, _ = oracle.quantize(x, oracle.MXFP4)
    assert scales.shape == (1, 1)
    assert oracle.e8m0_decode(int(scales[0, 0])) == g["mxfp4"]["scale"]
    y = oracle.dequantize(codes, scales, oracle.MXFP4)[0]
    assert np.array_equal(y[:8], np.array(g["mxfp4"]["reconstruction_printed"], np.float32)), y[:8]
    assert np.all(y[8:] == 0)
    # the scaled values the page prints (x / s) round onto the same grid points
    sv = np.array(g["mxfp4"]["scaled_values_printed"])
    assert np.allclose(sv, np.array(g["values"]) / g["mxfp4"]["scale"], atol=1e-9)


def check_worked_example_nvfp4():
    g = _golden("vs_worked_example.json")
    x = np.zeros(16, np.float32)
    x[:8] = g["values"]
    codes, scales, ts = oracle.quantize(x, oracle.NVFP4)
    assert ts == np.float32(2.6) / np.float32(2688.0)
    s = oracle.e4m3_decode(int(scales[0, 0])) * float(ts)
    assert scales[0, 0] == 0x7E                              # 2.6 maps onto 6 exactly
    assert abs(s - g["nvfp4"]["scale_approx"]) < 5e-4
    y = oracle.dequantize(codes, scales, oracle.NVFP4, ts)[0]
    d = g["nvfp4"]["printed_decimals"]
    assert np.array_equal(np.round(y[:8].astype(np.float64), d),
                          np.array(g["nvfp4"]["reconstruction_printed"])), y[:8]
    assert np.all(y[8:] == 0)
    # the printed scaled values (x / s, 2 decimals) round to the grid points used
    sv = np.array(g["nvfp4"]["scaled_values_printed"])
    assert np.allclose(np.array(g["values"]) / s, sv, atol=0.006)


def check_emulation_table():
    g = _golden("vs_emulation_table.json")
    r = np.random.default_rng(0)
    n = 1 << 20
    gauss = r.standard_normal(n)
    outl = r.standard_normal(n) * (1 + 9 * (r.random(n) < 0.002))
    data = {"gaussian": gauss, "outliers": outl}
    for row in g["rows"]:
        x = data[row["data"]]
        fmt = oracle.MXFP4 if row["format"] == "MXFP4" else oracle.NVFP4
        c, s, ts = oracle.quantize(x.astype(np.float32), fmt)
        y = oracle.dequantize(c, s, fmt, ts).reshape(-1)
        # MSE and SQNR from the oracle's error sums (the input is the fp32 copy
        # the oracle quantized; the float64 -> fp32 cast moves no printed digit)
        se, sx, _, _ = oracle.error_sums(x.astype(np.float32), y)
        mse = se / n
        sqnr = 10 * np.log10(sx / se)
        assert round(mse, 5) == row["mse"], (row, mse)
        assert round(sqnr, 2) == row["sqnr_db"], (row, sqnr)


# ------------------------------------------------------------------ Hadamard
def check_hadamard_matches_sylvester():
    for n in (16, 32):
        H = scipy.linalg.hadamard(n).astype(np.float64)
        eye = np.eye(n, dtype=np.float32)
        R = oracle.rotate(eye, n).astype(np.float64)          # row j = e_j H / sqrt(n)
        assert np.allclose(R, H / np.sqrt(n), rtol=0, atol=1e-7), n
        assert np.allclose(R @ R.T, np.eye(n), atol=1e-6)
        ones = np.ones((1, n), np.float32)
        v = oracle.rotate(ones, n)[0]
        assert abs(v[0] - np.sqrt(n)) < 1e-5 and np.all(np.abs(v[1:]) < 1e-6)


def check_hadamard_involution_and_norm():
    x = workloads.laplace(workloads.rng(13, 13), 64 * 96, 1.0).astype(np.float32).reshape(64, 96)
    for n in (16, 32):
        y = oracle.rotate(x, n)
        z = oracle.rotate(y, n)
        assert np.allclose(z, x, rtol=0, atol=1e-5)
        # per block norm preservation
        xb = x.reshape(64, -1, n).astype(np.float64)
        yb = y.reshape(64, -1, n).astype(np.float64)
        assert np.allclose((xb ** 2).sum(-1), (yb ** 2).sum(-1), rtol=1e-6)
        # the transform is block-local: a change in block b only moves block b
        x2 = x.copy()
        x2[:, 5] += 1.0
        d = np.abs(oracle.rotate(x2, n) - y) > 0
        assert not d[:, n:].any() and d[:, :n].all()


# --------------------------------------------------------------- quantizer
def _bf16_f32(bits):
    return workloads.bf16_bits_to_f32(bits)


def check_mx_idempotent():
    for x in (workloads.cfg1_tensor(3),
              _bf16_f32(workloads.cfg2_tensor("laplace", 3, rows=64, cols=512)),
              _bf16_f32(workloads.cfg2_tensor("gauss", 4, rows=64, cols=512))):
        for rot in (False, True):
            c, s, _ = oracle.quantize(x, oracle.MXFP4, rotate=rot)
            y = oracle.dequantize(c, s, oracle.MXFP4)
            c2, s2, _ = oracle.quantize(y, oracle.MXFP4)
            assert np.array_equal(c, c2) and np.array_equal(s, s2)


def check_nv_idempotent_on_normal_scales():
    x = _bf16_f32(workloads.cfg2_tensor("laplace", 5, rows=64, cols=512))
    for rot in (False, True):
        c, s, ts = oracle.quantize(x, oracle.NVFP4, rotate=rot)
        y = oracle.dequantize(c, s, oracle.NVFP4, ts)
        c2, s2, _ = oracle.quantize(y, oracle.NVFP4, ts=ts)
        normal = s >= 0x08
        assert normal.mean() > 0.9
        assert np.array_equal(s[normal], s2[normal])
        cb = c.reshape(c.shape[0], -1, 8)
        cb2 = c2.reshape(c.shape[0], -1, 8)
        assert np.array_equal(cb[normal], cb2[normal])


def check_invariants():
    x = _bf16_f32(workloads.cfg2_tensor("laplace", 6, rows=128, cols=1024))
    # MX: every nonzero block whose exponent is not clamped holds a code of
    # magnitude 4 or 6 (the scaled block maximum lies in [4, 8)).
    c, s, _ = oracle.quantize(x, oracle.MXFP4)
    mags = np.stack([c & 7, c >> 4 & 7], -1).reshape(c.shape[0], -1, 32)
    top = mags.max(-1)
    live = s > 0
    assert np.all(np.isin(top[live], [6, 7]))
    # scale codes are monotone in the block amax
    amax = np.abs(x.reshape(x.shape[0], -1, 32)).max(-1).reshape(-1)
    order = np.argsort(amax, kind="stable")
    assert np.all(np.diff(s.reshape(-1)[order].astype(int)) >= 0)
    # NV: the block holding the tensor amax gets scale code 0x7E (448) and an
    # element of magnitude 6; every scale code is <= 0x7E.
    c, s, ts = oracle.quantize(x, oracle.NVFP4)
    assert ts == np.float32(np.abs(x).max()) / np.float32(2688.0)
    flat = np.abs(x).reshape(x.shape[0], -1, 16)
    r, b = np.unravel_index(np.argmax(flat.max(-1)), flat.shape[:2])
    assert s[r, b] == 0x7E and s.max() == 0x7E
    blk = np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1, 16)[r, b]
    assert (blk & 7).max() == 7
    amax = flat.max(-1).reshape(-1)
    order = np.argsort(amax, kind="stable")
    assert np.all(np.diff(s.reshape(-1)[order].astype(int)) >= 0)


def check_brute_force_codes_tiny_blocks():
    """At a fixed scale, the code vector that minimises the block SSE over all
    16^n candidates is the element-wise nearest grid point; the oracle's codes
    must be a minimiser (and equal to it wherever the minimiser is unique)."""
    g = workloads.rng(14, 14)
    allv = np.array([oracle.e2m1_decode(c) for c in range(16)])
    for trial in range(60):
        n = 3
        x = g.laplace(0, 1, n).astype(np.float32)
        xb = np.zeros(32, np.float32)
        xb[:n] = x
        c, s, _ = oracle.quantize(xb, oracle.MXFP4)
        sv = oracle.e8m0_decode(int(s[0, 0]))
        codes = np.stack([c[0] & 15, c[0] >> 4], -1).reshape(-1)[:n]
        # brute force over every code vector
        grid = np.array(np.meshgrid(*[np.arange(16)] * n, indexing="ij")).reshape(n, -1)
        recon = allv[grid] * sv
        sse = ((recon - x[:, None].astype(np.float64)) ** 2).sum(0)
        best = sse.min()
        mine = ((allv[codes] * sv - x.astype(np.float64)) ** 2).sum()
        assert mine <= best * (1 + 1e-12) + 1e-300, (x, codes)
        # the absmax exponent is never worse than saturating everything
        assert mine <= ((x.astype(np.float64)) ** 2).sum() + 1e-12


def check_absmax_scale_vs_best_scale():
    """The absmax exponent is within one step of the SSE-optimal E8M0 exponent on
    Laplace blocks, and the optimum is below absmax+2 (the scale that maps the
    block maximum below 4 only loses resolution)."""
    g = workloads.rng(15, 15)
    allv = np.array([oracle.e2m1_decode(c) for c in range(8)])
    for _ in range(200):
        x = g.laplace(0, 1, 32).astype(np.float32)
        c, s, _ = oracle.quantize(x, oracle.MXFP4)
        e0 = int(s[0, 0]) - 127
        sses = {}
        for e in range(e0 - 3, e0 + 4):
            sv = 2.0 ** e
            a = np.abs(x) / sv
            q = allv[np.abs(np.minimum(a, 6)[:, None] - allv).argmin(-1)]
            sses[e] = ((np.sign(x) * q * sv - x) ** 2).sum()
        best = min(sses, key=sses.get)
        assert best in (e0, e0 + 1), (e0, sses)


# ------------------------------------------------------ INT4 element formats
def check_int4_codec():
    """MXINT4 / NVINT4 element ([MRGPTQ]: the MX / NV formats with an INT4
    element): a two's-complement nibble decodes to -8 .. 7; encoding is the
    nearest integer (numpy's rint: ties to even) clipped to +-7, stored as
    value & 15 (so -8 is never produced and zero has one code)."""
    vals = np.array([oracle.int4_decode(c) for c in range(16)])
    assert np.array_equal(vals, np.array(list(range(8)) + list(range(-8, 0)), dtype=float)), vals
    g = workloads.rng(42, 42)
    ints = np.arange(-9, 10, dtype=np.float64)
    mids = ints[:-1] + 0.5
    probe = [ints, mids, g.uniform(-12, 12, 20000), np.array([1e30, -1e30, 0.0, -0.0, 7.4999, 7.5])]
    for arr in (ints, mids):
        f = arr.astype(np.float32)
        probe += [np.nextafter(f, np.float32(-1e9)), np.nextafter(f, np.float32(1e9))]
    q = np.concatenate(probe).astype(np.float32)
    codes = oracle.int4_encode_array(q)
    ref = np.clip(np.rint(q.astype(np.float64)), -7, 7).astype(np.int64) & 15
    bad = np.nonzero(codes != ref)[0]
    assert bad.size == 0, (q[bad[:5]], codes[bad[:5]], ref[bad[:5]])
    assert not np.any(codes == 8)
    assert oracle.int4_encode(-0.0) == 0 and oracle.int4_encode(-0.4) == 0
    assert oracle.int4_encode(2.5) == 2 and oracle.int4_encode(-3.5) == (-4 & 15)


def check_int4_worked_blocks():
    """Hand-checked blocks.  MXINT4: [7, -3, 2, 0.5, 0 ...] has floor(log2 7) - 2
    = 0, scale 2^0, codes 7, -3, 2, 0 (0.5 ties to even).  NVINT4: a tensor whose
    maximum is 7 has ts = 7 / 3136, the block holding it takes E4M3 code 0x7E
    (448) and codes 7, -3, 1, 3 for [7, -3, 1.2, 2.6]."""
    x = np.zeros(32, np.float32)
    x[:4] = [7.0, -3.0, 2.0, 0.5]
    c, s, _ = oracle.quantize(x, oracle.MXINT4)
    assert s[0, 0] == 127, s
    codes = np.stack([c[0] & 15, c[0] >> 4], -1).reshape(-1)
    assert list(codes[:5]) == [7, 13, 2, 0, 0], codes[:5]
    y = oracle.dequantize(c, s, oracle.MXINT4)
    assert list(y[0, :4]) == [7.0, -3.0, 2.0, 0.0]
    xn = np.zeros(32, np.float32)
    xn[:4] = [7.0, -3.0, 1.2, 2.6]
    xn[16:18] = [0.7, -0.35]
    c, s, ts = oracle.quantize(xn, oracle.NVINT4)
    assert ts == np.float32(np.float32(7.0) / np.float32(3136.0))
    assert s[0, 0] == 0x7E, s
    codes = np.stack([c[0] & 15, c[0] >> 4], -1).reshape(-1)
    assert list(codes[:4]) == [7, 13, 1, 3], codes[:4]
    # second block: amax 0.7 -> (0.7 / 7) / ts = 44.8 -> the nearest E4M3 value
    e4 = _e4m3_values_from_definition()
    t = (np.float32(0.7) / np.float32(7.0)) / ts
    assert e4[s[0, 1]] == _binade_rne_e4m3(np.array([t], np.float32))[0]


def check_int4_invariants():
    """MXINT4: every block not clamped at the smallest scale has a code of
    magnitude 4..7 (the scaled maximum lies in [4, 8)); NVINT4: the block that
    holds the tensor maximum has scale code 0x7E and a code of magnitude 7;
    neither format produces the pattern 0x8; MXINT4 is idempotent
    (Q(D(Q(x))) = Q(x))."""
    x = workloads.laplace(workloads.rng(43, 43), 64 * 512, 1.0).astype(np.float32).reshape(64, 512)
    for rot in (False, True):
        c, s, _ = oracle.quantize(x, oracle.MXINT4, rot)
        v = np.stack([c & 15, c >> 4], -1).reshape(64, -1).astype(np.int64)
        sv = np.where(v >= 8, v - 16, v)
        assert not np.any(v == 8)
        mx = np.abs(sv).reshape(64, -1, 32).max(-1)
        assert np.all((mx >= 4) & (mx <= 7)), np.unique(mx)
        if not rot:
            y = oracle.dequantize(c, s, oracle.MXINT4)
            c2, s2, _ = oracle.quantize(y, oracle.MXINT4)
            assert np.array_equal(c2, c) and np.array_equal(s2, s)
        c, s, ts = oracle.quantize(x, oracle.NVINT4, rot)
        v = np.stack([c & 15, c >> 4], -1).reshape(64, -1).astype(np.int64)
        assert not np.any(v == 8)
        y = x if not rot else _block_values(x, 16, True).reshape(64, -1)
        r, b = np.unravel_index(np.abs(y).argmax(), y.shape)
        assert s[r, b // 16] == 0x7E
        blk = np.where(v[r, (b // 16) * 16:(b // 16) * 16 + 16] >= 8,
                       v[r, (b // 16) * 16:(b // 16) * 16 + 16] - 16, v[r, (b // 16) * 16:(b // 16) * 16 + 16])
        assert np.abs(blk).max() == 7


def check_int4_error_ordering():
    """[MRGPTQ]'s error analysis predicts that NVINT4 profits from the block
    Hadamard and beats the other formats: on Laplace data NVINT4 + H16 has the
    lowest NMSE of {MXFP4, NVFP4, MXINT4, NVINT4} x {plain, rotated}, below
    plain NVINT4; on Gaussian data NVINT4 is below NVFP4 (uniform grid)."""
    g = workloads.rng(44, 44)
    lap = workloads.laplace(g, 256 * 1024, 1.0).astype(np.float32).reshape(256, 1024)
    gau = workloads.normal(g, 256 * 1024, 1.0).astype(np.float32).reshape(256, 1024)

    def nm(x, fmt, rot):
        c, s, t = oracle.quantize(x, fmt, rot)
        y = oracle.dequantize(c, s, fmt, t, inverse_rotate=rot).astype(np.float64)
        return ((x - y) ** 2).sum() / (x.astype(np.float64) ** 2).sum()

    res = {(f, r): nm(lap, f, r) for f in (0, 1, 2, 3) for r in (False, True)}
    best = min(res, key=res.get)
    assert best == (oracle.NVINT4, True), res
    assert res[(oracle.NVINT4, True)] < res[(oracle.NVINT4, False)]
    assert nm(gau, oracle.NVINT4, False) < nm(gau, oracle.NVFP4, False)


def check_gemm_int4_closed_forms():
    """MXINT4 with every scale code 127 is an integer dot product (numpy int64
    matmul of the two's-complement nibbles); NVINT4 sums int x E4M3 products
    (E4M3 values from the definition) and multiplies by a_ts * b_ts."""
    g = workloads.rng(45, 45)
    M, N, K = 5, 7, 64
    ac = g.integers(0, 256, (M, K // 2)).astype(np.uint8)
    bc = g.integers(0, 256, (N, K // 2)).astype(np.uint8)

    def ints(c):
        v = np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1).astype(np.int64)
        return np.where(v >= 8, v - 16, v)

    ones = np.full((M, K // 32), 127, np.uint8), np.full((N, K // 32), 127, np.uint8)
    y, ab = oracle.gemm_full(oracle.MXINT4, K, ac, ones[0], 0.0, bc, ones[1], 0.0)
    assert np.array_equal(y, (ints(ac) @ ints(bc).T).astype(np.float64))
    assert np.array_equal(ab, (np.abs(ints(ac)) @ np.abs(ints(bc)).T).astype(np.float64))
    e4 = _e4m3_values_from_definition()
    asc = g.integers(0x20, 0x70, (M, K // 16)).astype(np.uint8)
    bsc = g.integers(0x20, 0x70, (N, K // 16)).astype(np.uint8)
    ats, bts = np.float32(0.013), np.float32(2.5e-3)
    y, _ = oracle.gemm_full(oracle.NVINT4, K, ac, asc, ats, bc, bsc, bts)
    av = ints(ac) * np.repeat(e4[asc], 16, axis=1)
    bv = ints(bc) * np.repeat(e4[bsc], 16, axis=1)
    ref = (av @ bv.T) * (float(ats) * float(bts))
    assert np.allclose(y, ref, rtol=1e-13, atol=0)


# ------------------------------------- rotation and rounding variants
KAT = _golden("philox4x32_10_kat.json")
MASK = 0x0123456789ABCDEF0FEDCBA987654321


def check_philox_known_answers():
    """Philox4x32-10, the counter-based generator behind stochastic rounding,
    reproduces its published known-answer vectors."""
    for v in KAT["vectors"]:
        out = oracle.philox4x32_10([int(c, 16) for c in v["ctr"]], [int(k, 16) for k in v["key"]])
        assert [int(o) for o in out] == [int(o, 16) for o in v["out"]], (v, [hex(o) for o in out])


def check_signed_rotation_is_the_matrix_product():
    """Rotation groups of 16 .. 128 with a random sign diagonal D: the oracle's
    y equals (x D) H_n / sqrt(n) from scipy's Sylvester matrix (double, then
    fp32) up to one ulp in at most 1e-4 of the elements; the inverse returns x;
    an all-zero mask is the plain transform."""
    g = workloads.rng(47, 47)
    x = g.normal(0, 1, (8, 256)).astype(np.float32)
    for n in (16, 32, 64, 128):
        bits = np.array([(MASK >> i) & 1 for i in range(n)])
        d = np.where(bits == 1, -1.0, 1.0)
        ref = ((x.astype(np.float64).reshape(-1, n) * d) @ scipy.linalg.hadamard(n) / np.sqrt(n))
        ref = ref.astype(np.float32).reshape(x.shape)
        y = oracle.rotate_signed(x, n, MASK)
        ulp = np.abs(y.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1 and (ulp > 0).mean() <= 1e-4, (n, ulp.max())
        back = oracle.rotate_signed(y, n, MASK, inverse=True)
        assert np.allclose(back, x, rtol=0, atol=1e-5 * np.abs(x).max()), n
        assert np.array_equal(oracle.rotate_signed(x, n, 0), oracle.rotate(x, n))


def check_mx_rotation_sizes():
    """MXFP4 with a 64- or 128-point rotation quantizes the rotated values with
    the usual 32-element scales: equal to quantizing rotate_signed(x) without a
    rotation, and dequantize with the inverse rotation gives back x up to the
    quantization error."""
    x = workloads.laplace(workloads.rng(48, 48), 32 * 512, 1.0).astype(np.float32).reshape(32, 512)
    for n in (64, 128):
        c, s, _ = oracle.quantize_spec(x, oracle.MXFP4, rot_n=n, signs=MASK)
        c2, s2, _ = oracle.quantize(oracle.rotate_signed(x, n, MASK), oracle.MXFP4)
        assert np.array_equal(c, c2) and np.array_equal(s, s2), n
        y = oracle.dequantize_rot(c, s, oracle.MXFP4, 0.0, rot_n=n, signs=MASK)
        assert ((y - x) ** 2).sum() / (x ** 2).sum() < 0.02


def check_stochastic_rounding_definition():
    """Stochastic rounding ([VS]: up or down with probability proportional to
    proximity): grid points never move; between neighbours lo < a < hi the value
    rounds up exactly when u < (a - lo) / (hi - lo); saturation at 6; the sign
    bit is kept."""
    enc = oracle.e2m1_encode_sr
    for c in range(8):
        v = oracle.e2m1_decode(c)
        for u in (0.0, 0.3, 0.999):
            assert enc(v, u) == c and enc(-v, u) == (8 | c)
    assert enc(0.75, 0.49) == 2 and enc(0.75, 0.5) == 1          # p = 1/2
    assert enc(2.25, 0.2) == 5 and enc(2.25, 0.25) == 4          # p = 1/4 between 2 and 3
    assert enc(5.0, 0.4999) == 7 and enc(5.0, 0.5) == 6          # between 4 and 6
    assert enc(-0.3, 0.1) == 0x9 and enc(-0.3, 0.9) == 0x8       # p = 0.6 between 0 and 0.5
    assert enc(7.5, 0.0) == 7 and enc(1e30, 0.9) == 7


def check_stochastic_rounding_stream():
    """Tensor-level stochastic rounding: element e uses word e % 4 of
    Philox4x32-10(counter = e / 4, key = seed); with seed 0 the first four
    elements see the first known-answer vector.  Every code is a neighbour of
    the quotient; the rounding is unbiased on a 0.3 plateau; the same seed
    repeats, another seed changes the codes."""
    x = np.zeros((64, 32 * 16), np.float32)
    x[0, :4] = [0.75, 6.0, 0.75, 2.5]         # scale 2^0; p = 1/2, grid, 1/2, 1/2
    c, s, _ = oracle.quantize_spec(x, oracle.MXFP4, rounding=oracle.ROUND_STOCHASTIC, seed=(0, 0))
    u = [int(w, 16) >> 8 for w in KAT["vectors"][0]["out"]]
    u = [v * 2.0 ** -24 for v in u]           # 0.399, 0.880, 0.736, 0.607
    codes = np.stack([c[0] & 15, c[0] >> 4], -1).reshape(-1)[:4]
    want = [2 if u[0] < 0.5 else 1, 7, 2 if u[2] < 0.5 else 1, 5 if u[3] < 0.5 else 4]
    assert list(codes) == want, (list(codes), want)
    # a plateau of 0.3 (p = 0.6 of rounding up to 0.5) next to a 6 in every block
    y = np.full((64, 32 * 16), 0.3, np.float32)
    y[:, ::16] = 6.0
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        c1, s1, t1 = oracle.quantize_spec(y, fmt, rounding=oracle.ROUND_STOCHASTIC, seed=(7, 9))
        d = oracle.dequantize(c1, s1, fmt, t1)
        scale = d[:, ::16].mean() / 6.0
        vals = np.round(np.delete(d, np.s_[::16], axis=1) / scale, 5)   # NVFP4: s = 448 ts ~ 1
        assert set(np.unique(vals)) <= {0.0, 0.5}, np.unique(vals)
        n = vals.size
        assert abs(vals.mean() - 0.3) < 5 * 0.5 * np.sqrt(0.24 / n), vals.mean()
        c2, _, _ = oracle.quantize_spec(y, fmt, rounding=oracle.ROUND_STOCHASTIC, seed=(7, 9))
        c3, _, _ = oracle.quantize_spec(y, fmt, rounding=oracle.ROUND_STOCHASTIC, seed=(8, 9))
        assert np.array_equal(c1, c2) and (c1 != c3).mean() > 0.3
    # codes are neighbours of the quotient on generic data
    z = workloads.laplace(workloads.rng(49, 49), 16 * 512, 1.0).astype(np.float32).reshape(16, 512)
    c, s, _ = oracle.quantize_spec(z, oracle.MXFP4, rounding=oracle.ROUND_STOCHASTIC, seed=(1, 2))
    cn, sn, _ = oracle.quantize(z, oracle.MXFP4)
    assert np.array_equal(s, sn)
    q = z / np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    full = np.concatenate([-GRID[:0:-1], GRID])
    v = np.stack([c & 15, c >> 4], -1).reshape(16, -1)
    val = np.where(v & 8, -GRID[v & 7], GRID[v & 7])
    qc = np.clip(q, -6, 6)
    lo = full[np.searchsorted(full, qc, side="right") - 1]
    hi = full[np.minimum(np.searchsorted(full, qc, side="left"), full.size - 1)]
    assert np.all((val == lo) | (val == hi))


def check_two_dimensional_nvfp4_blocks():
    """NVFP4 16x16 weight blocks ([VS] "Two-dimensional weight scaling"): the 16
    rows of a tile share the scale E4M3((tile max / 6) / ts) (E4M3 rounding from
    the format definition), a tile and its transpose get the same scale, and
    the codes are nearest grid points at that scale.  A partial last tile
    (40 rows) uses the rows it has."""
    e4 = _e4m3_values_from_definition()
    w = workloads.laplace(workloads.rng(50, 50), 64 * 256, 1.0).astype(np.float32).reshape(64, 256)
    c, s, ts = oracle.quantize_spec(w, oracle.NVFP4, block_rows=16)
    ct, st, tst = oracle.quantize_spec(np.ascontiguousarray(w.T), oracle.NVFP4, block_rows=16)
    assert ts == tst
    tiles = np.abs(w).reshape(4, 16, 16, 16).max(axis=(1, 3))          # [row tile, col block]
    want = np.searchsorted(e4, _binade_rne_e4m3((tiles.astype(np.float32) / np.float32(6)) / ts))
    assert np.array_equal(s.reshape(4, 16, 16), np.repeat(want[:, None, :], 16, axis=1))
    assert np.array_equal(st.reshape(16, 16, 4), np.repeat(want.T[:, None, :], 16, axis=1))
    y = oracle.dequantize(c, s, oracle.NVFP4, ts).astype(np.float64)
    sv = np.repeat((e4[s].astype(np.float32) * np.float32(ts)).astype(np.float64), 16, axis=1)
    best = np.abs(np.abs(w)[..., None] - GRID[None, None, :] * sv[..., None]).min(-1)
    # y rounds e2m1 * e4m3 * ts once: within 2^-22 |w| of the brute-force distance
    assert np.all(np.abs(np.abs(y - w) - best) <= 2.0 ** -22 * np.abs(w) + 1e-30)
    c4, s4, _ = oracle.quantize_spec(w[:40], oracle.NVFP4, block_rows=16, ts=ts)
    assert np.array_equal(s4[:32], s[:32])
    last = np.abs(w[32:40]).reshape(8, 16, 16).max(axis=(0, 2))
    assert np.array_equal(s4[32], np.searchsorted(e4, _binade_rne_e4m3((last / np.float32(6)) / ts)))


# ------------------------------------------------ scale search (MSE, 4/6)
MX_WINDOW = (0, 1)
NV_WINDOW = (0, 1, -1, 2, -2, 3, 4, 5, 6)


def _block_values(x: np.ndarray, G: int, rotate: bool) -> np.ndarray:
    """[blocks, G] float64 of the values the block scales see: x itself, or the
    block Hadamard (scipy's Sylvester matrix / sqrt(G)) rounded to fp32."""
    y = x.astype(np.float64).reshape(-1, G)
    if rotate:
        y = (y @ (scipy.linalg.hadamard(G) / np.sqrt(G))).astype(np.float32).astype(np.float64)
    return y


def _best_sse_at(y: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Brute force: for blocks y [nb, G] and scales s [nb, C] (float64), the
    smallest possible squared error of each block at each scale, every element
    taking the best of the eight grid magnitudes (its sign is free)."""
    a = np.abs(y)[:, None, :, None]                           # nb, 1, G, 1
    cand = GRID[None, None, None, :] * s[:, :, None, None]    # nb, C, 1, 8
    return ((a - cand) ** 2).min(-1).sum(-1)                  # nb, C


def _scale_values(fmt, codes, ts):
    if fmt == oracle.MXFP4:
        return np.exp2(codes.astype(np.float64) - 127)
    e4 = _e4m3_values_from_definition()
    return (e4[codes].astype(np.float32) * np.float32(ts)).astype(np.float64)


def _search_inputs():
    g = workloads.rng(41, 41)
    lap = workloads.laplace(g, 32 * 1024, 1.0).astype(np.float32).reshape(32, 1024)
    gau = workloads.normal(g, 32 * 1024, 0.02).astype(np.float32).reshape(32, 1024)
    return [("laplace", lap), ("gauss", gau)]


def check_mse_scale_is_the_window_optimum():
    """FP4_SCALE_MSE ("MSE scale optimization", "format-specific scale search";
    the best scale need not put the block maximum on 6): each block's scale code
    is the absmax code c0 or one of its window neighbours (MXFP4 c0, c0+1;
    NVFP4 c0-2 .. c0+6), its squared error (brute force over the grid, double)
    is the smallest in the window, and where the window minimum is clear by
    1e-4 it is that code exactly.  Codes at the chosen scale are nearest grid
    points.  The tensor scale is the absmax rule's."""
    for name, x in _search_inputs():
        for fmt in (oracle.MXFP4, oracle.NVFP4):
            G = oracle.BLOCK[fmt]
            win = np.array(MX_WINDOW if fmt == oracle.MXFP4 else NV_WINDOW)
            top = 254 if fmt == oracle.MXFP4 else 0x7E
            for rot in (False, True):
                _, s0, ts0 = oracle.quantize(x, fmt, rot)
                c, s, ts = oracle.quantize(x, fmt, rot, rule=oracle.SCALE_MSE)
                assert ts == ts0, (name, fmt, rot)
                y = _block_values(x, G, rot)
                c0 = s0.reshape(-1).astype(np.int64)
                ch = s.reshape(-1).astype(np.int64)
                cand = c0[:, None] + win[None, :]
                valid = (cand >= 0) & (cand <= top)
                e = _best_sse_at(y, _scale_values(fmt, np.clip(cand, 0, top), ts))
                e = np.where(valid, e, np.inf)
                assert np.all(np.any(cand == ch[:, None], axis=1)), (name, fmt, rot)
                e_ch = _best_sse_at(y, _scale_values(fmt, ch[:, None], ts))[:, 0]
                best = e.min(1)
                assert np.all(e_ch <= best * (1 + 1e-5) + 1e-300), (name, fmt, rot)
                srt = np.sort(e, 1)
                clear = srt[:, 1] > srt[:, 0] * (1 + 1e-4)
                arg = cand[np.arange(cand.shape[0]), e.argmin(1)]
                assert np.array_equal(ch[clear], arg[clear]), (name, fmt, rot)
                # the element codes are the nearest grid points at that scale (the
                # dequantized NVFP4 value rounds e2m1 * e4m3 * ts once: a 2^-24
                # relative change of each reconstruction)
                xh = oracle.dequantize(c, s, fmt, ts).astype(np.float64).reshape(-1, G)
                got = ((xh - y) ** 2).sum(1)
                slack = 2.0 ** -22 * np.sqrt(e_ch * (y ** 2).sum(1)) + 1e-300
                assert np.all(np.abs(got - e_ch) <= 1e-9 * e_ch + slack), (name, fmt, rot)
                # and the search lowers the error of the tensor
                c_a, s_a, _ = oracle.quantize(x, fmt, rot)
                xa = oracle.dequantize(c_a, s_a, fmt, ts).astype(np.float64).reshape(-1, G)
                assert got.sum() < ((xa - y) ** 2).sum(), (name, fmt, rot)


def check_mse_window_holds_the_global_optimum():
    """The window is wide enough: over every representable scale code the
    squared-error optimum lies inside it for at least 99.9 % of Laplace and
    Gaussian blocks (plain and rotated)."""
    for name, x in _search_inputs():
        for fmt in (oracle.MXFP4, oracle.NVFP4):
            G = oracle.BLOCK[fmt]
            win = np.array(MX_WINDOW if fmt == oracle.MXFP4 else NV_WINDOW)
            for rot in (False, True):
                _, s0, ts = oracle.quantize(x, fmt, rot)
                y = _block_values(x, G, rot)
                c0 = s0.reshape(-1).astype(np.int64)
                if fmt == oracle.MXFP4:
                    allc = np.clip(c0[:, None] + np.arange(-8, 9)[None, :], 0, 254)
                else:
                    allc = np.tile(np.arange(0x7F), (c0.size, 1))
                e = _best_sse_at(y, _scale_values(fmt, allc, ts))
                opt = allc[np.arange(allc.shape[0]), e.argmin(1)] - c0
                inside = np.isin(opt, win).mean()
                assert inside >= 0.999, (name, fmt, rot, inside)


def check_four_over_six():
    """FP4_SCALE_FOUR_OVER_SIX (NVFP4; "Four Over Six": some blocks map their
    maximum to 4 instead of 6): the scale code is c6 = E4M3((amax/6)/ts) or
    c4 = E4M3((amax/4)/ts) (E4M3 rounding from the format definition), the one
    with the smaller squared error where the two differ by 1e-4, and the
    tensor error is below the absmax rule's."""
    e4 = _e4m3_values_from_definition()
    for name, x in _search_inputs():
        for rot in (False, True):
            _, s6, ts = oracle.quantize(x, oracle.NVFP4, rot)
            c, s, ts2 = oracle.quantize(x, oracle.NVFP4, rot, rule=oracle.SCALE_FOUR_OVER_SIX)
            assert ts2 == ts
            y = _block_values(x, 16, rot)
            amax = np.abs(y).max(1).astype(np.float32)
            t4 = (amax / np.float32(4)) / np.float32(ts)
            c4 = np.searchsorted(e4, _binade_rne_e4m3(t4))
            c6 = s6.reshape(-1).astype(np.int64)
            assert np.array_equal(e4[c6], _binade_rne_e4m3((amax / np.float32(6)) / np.float32(ts)))
            ch = s.reshape(-1).astype(np.int64)
            assert np.all((ch == c6) | (ch == c4)), (name, rot)
            e = _best_sse_at(y, _scale_values(oracle.NVFP4, np.stack([c6, c4], 1), ts))
            clear = np.abs(e[:, 0] - e[:, 1]) > 1e-4 * np.maximum(e[:, 0], e[:, 1])
            want = np.where(e[:, 1] < e[:, 0], c4, c6)
            assert np.array_equal(ch[clear], want[clear]), (name, rot)
            assert (c4 != c6).mean() > 0.9
            xh = oracle.dequantize(c, s, oracle.NVFP4, ts).astype(np.float64).reshape(-1, 16)
            xa = oracle.dequantize(*oracle.quantize(x, oracle.NVFP4, rot)[:2], oracle.NVFP4, ts)
            assert ((xh - y) ** 2).sum() < ((xa.astype(np.float64).reshape(-1, 16) - y) ** 2).sum()


def check_scale_search_ties_keep_the_absmax_code():
    """Equal errors keep the absmax code: a block exact at both 2^e0 and
    2^(e0+1) (MXFP4), all-zero blocks, and an NVFP4 block exact at its absmax
    scale keep c0 under every rule."""
    x = np.zeros((2, 64), np.float32)
    x[0, :4] = [4.0, 2.0, -1.0, 2.0]          # exact at 2^0 and at 2^1
    c, s, _ = oracle.quantize(x, oracle.MXFP4, rule=oracle.SCALE_MSE)
    assert s[0, 0] == 127 and s[0, 1] == 0 and np.all(s[1] == 0), s
    xn = np.zeros((2, 32), np.float32)
    xn[0, :3] = [6.0, 3.0, -1.5]                 # ts = 6/2688: c0 = 448 exact
    for rule in (oracle.SCALE_MSE, oracle.SCALE_FOUR_OVER_SIX):
        c, s, ts = oracle.quantize(xn, oracle.NVFP4, rule=rule)
        assert s[0, 0] == 0x7E and s[0, 1] == 0 and np.all(s[1] == 0), (rule, s)
        assert np.all(c[1] == 0)


def check_directional_rotation():
    """Under RTN, a group-sized Hadamard lowers MXFP4 error on Laplace data and
    raises NVFP4 error ("rotations improve MXFP4 accuracy, but hurt NVFP4")."""
    x = workloads.laplace(workloads.rng(16, 16), 1 << 18, 1.0).astype(np.float32).reshape(256, 1024)
    res = {}
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        for rot in (False, True):
            c, s, ts = oracle.quantize(x, fmt, rotate=rot)
            y = oracle.dequantize(c, s, fmt, ts, inverse_rotate=rot)
            res[fmt, rot] = oracle.nmse(x, y)
    assert res[oracle.MXFP4, True] < res[oracle.MXFP4, False] * 0.95, res
    assert res[oracle.NVFP4, True] > res[oracle.NVFP4, False] * 1.02, res


def check_nmse_domains_agree():
    """The rotation is orthogonal, so the error measured in the rotated domain
    equals the error in the original domain (eq. (2) of the portable-FP4 page)."""
    x = _bf16_f32(workloads.cfg3_tensor(7, rows=32, cols=1024))
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        c, s, ts = oracle.quantize(x, fmt, rotate=True)
        y_rot = oracle.dequantize(c, s, fmt, ts)
        y_orig = oracle.dequantize(c, s, fmt, ts, inverse_rotate=True)
        xr = oracle.rotate(x, oracle.BLOCK[fmt])
        a = oracle.nmse(xr, y_rot)
        b = oracle.nmse(x, y_orig)
        assert abs(a - b) <= 1e-5 * a, (a, b)
        assert 0 < oracle.cosine(x, y_orig) <= 1.0


def check_error_sums_closed_form():
    """Hand-computed sums: x = (3, 4, 0, -1), x^ = (0, 4, 1, -2)."""
    x = np.array([3, 4, 0, -1], np.float32)
    xh = np.array([0, 4, 1, -2], np.float32)
    se, sx, sxy, sy = oracle.error_sums(x, xh)
    assert (se, sx, sxy, sy) == (9 + 0 + 1 + 1, 9 + 16 + 0 + 1, 0 + 16 + 0 + 2, 0 + 16 + 1 + 4)
    assert oracle.nmse(x, xh) == 11 / 26
    assert abs(oracle.cosine(x, xh) - 18 / np.sqrt(26 * 21)) < 1e-15
    assert oracle.cosine(x, 2 * x) == 1.0


def check_zero_and_tiny_inputs():
    z = np.zeros((2, 64), np.float32)
    c, s, _ = oracle.quantize(z, oracle.MXFP4)
    assert np.all(c == 0) and np.all(s == 0)
    c, s, ts = oracle.quantize(z, oracle.NVFP4)
    assert ts == 0 and np.all(c == 0) and np.all(s == 0)
    assert np.all(oracle.dequantize(c, s, oracle.NVFP4, ts) == 0)
    # one zero block inside a live tensor
    x = np.zeros((1, 64), np.float32)
    x[0, 40] = 3.0
    c, s, ts = oracle.quantize(x, oracle.NVFP4)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[0, 2] == 0x7E
    c, s, _ = oracle.quantize(x, oracle.MXFP4)
    assert s[0, 0] == 0 and s[0, 1] == 126          # floor(log2 3) - 2 = -1
    # tiny values clamp the exponent at -127 and stay representable
    t = np.full((1, 32), 2.0 ** -130, np.float32)
    c, s, _ = oracle.quantize(t, oracle.MXFP4)
    assert s[0, 0] == 0
    y = oracle.dequantize(c, s, oracle.MXFP4)
    assert np.allclose(y, t, rtol=0.5)


# --------------------------------------------------------------------- GEMM
def _decode_codes(codes: np.ndarray) -> np.ndarray:
    """Signed grid values of packed codes (low nibble first), from the value
    set of the format definitions."""
    lo = codes & 15
    hi = codes >> 4
    c = np.stack([lo, hi], -1).reshape(codes.shape[0], -1)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def check_gemm_integer_closed_form():
    """K = 32 with every E8M0 code 127 (scale 1): twice every grid value is an
    integer, so y = (1/4) * (2A)(2B)^T exactly, in integer arithmetic."""
    g = workloads.rng(17, 17)
    M, N, K = 9, 7, 32
    ac = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = np.full((M, 1), 127, np.uint8)
    bsc = np.full((N, 1), 127, np.uint8)
    y, ab = oracle.gemm_full(oracle.MXFP4, K, ac, asc, 0, bc, bsc, 0)
    A2 = (2 * _decode_codes(ac)).astype(np.int64)
    B2 = (2 * _decode_codes(bc)).astype(np.int64)
    assert np.array_equal(y * 4, (A2 @ B2.T).astype(np.float64))
    assert np.array_equal(ab * 4, (np.abs(A2) @ np.abs(B2).T).astype(np.float64))


def check_gemm_block_scaled_closed_form():
    """Random E8M0 / E4M3 scales: y = sum over K-blocks of scaleA*scaleB times an
    integer block dot product (NVFP4: times tsA * tsB), computed block-wise in
    numpy from the format definitions; also y(A, B) = y(B, A)^T."""
    g = workloads.rng(18, 18)
    vals = _e4m3_values_from_definition()
    for fmt, G in ((oracle.MXFP4, 32), (oracle.NVFP4, 16)):
        M, N, K = 6, 5, 256
        ac = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
        bc = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
        if fmt == oracle.MXFP4:
            asc = g.integers(110, 140, (M, K // G), dtype=np.uint8)
            bsc = g.integers(110, 140, (N, K // G), dtype=np.uint8)
            sa = np.exp2(asc.astype(np.float64) - FMT["e8m0_bias"])
            sb = np.exp2(bsc.astype(np.float64) - FMT["e8m0_bias"])
            ta, tb = 0.0, 0.0
            gs = 1.0
        else:
            asc = g.integers(1, 127, (M, K // G), dtype=np.uint8)
            bsc = g.integers(1, 127, (N, K // G), dtype=np.uint8)
            sa, sb = vals[asc], vals[bsc]
            ta, tb = np.float32(0.0123), np.float32(3.5e-4)
            gs = float(ta) * float(tb)
        y, ab = oracle.gemm_full(fmt, K, ac, asc, ta, bc, bsc, tb)
        A2 = (2 * _decode_codes(ac)).astype(np.int64).reshape(M, K // G, G)
        B2 = (2 * _decode_codes(bc)).astype(np.int64).reshape(N, K // G, G)
        blockdot = np.einsum("mbg,nbg->mnb", A2, B2).astype(np.float64) / 4
        absdot = np.einsum("mbg,nbg->mnb", np.abs(A2), np.abs(B2)).astype(np.float64) / 4
        ref = (blockdot * sa[:, None, :] * sb[None, :, :]).sum(-1) * gs
        refa = (absdot * sa[:, None, :] * sb[None, :, :]).sum(-1) * abs(gs)
        assert np.allclose(y, ref, rtol=1e-12, atol=0), fmt
        assert np.allclose(ab, refa, rtol=1e-12, atol=0), fmt
        yt, _ = oracle.gemm_full(fmt, K, bc, bsc, tb, ac, asc, ta)
        assert np.array_equal(yt, y.T)
        # a row-local change in A moves only that row of Y
        ac2 = ac.copy()
        ac2[2, 3] ^= 0x11
        y2, _ = oracle.gemm_full(fmt, K, ac2, asc, ta, bc, bsc, tb)
        assert np.array_equal(np.delete(y2, 2, 0), np.delete(y, 2, 0))


def check_gemm_rotation_convention():
    """Q(X H) Q(W H)^T approximates X W^T: the block Hadamard is orthogonal, so
    rotating both operands along K leaves the product unchanged before
    quantization and close to it after."""
    X = _bf16_f32(workloads.gemm_activation(16, 512, 8))
    W = _bf16_f32(workloads.gemm_weight(24, 512, 8))
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        G = oracle.BLOCK[fmt]
        Xr = oracle.rotate(X, G).astype(np.float64)
        Wr = oracle.rotate(W, G).astype(np.float64)
        assert np.allclose(Xr @ Wr.T, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
        ca, sa, ta = oracle.quantize(X, fmt, rotate=True)
        cb, sb, tb = oracle.quantize(W, fmt, rotate=True)
        y, ab = oracle.gemm_full(fmt, 512, ca, sa, ta, cb, sb, tb)
        rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
        assert rel < 0.2, (fmt, rel)


def check_gemm_w4a16_integer_closed_form():
    """Weight-only GEMM, K = 32 with every E8M0 code 127: with integer
    activations, y = (1/2) * A (2B)^T exactly in integer arithmetic."""
    g = workloads.rng(19, 19)
    M, N, K = 5, 7, 32
    A = g.integers(-9, 10, (M, K)).astype(np.float32)
    bc = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bsc = np.full((N, 1), 127, np.uint8)
    y, ab = oracle.gemm_w4a16_full(oracle.MXFP4, K, A, bc, bsc, 0.0)
    B2 = (2 * _decode_codes(bc)).astype(np.int64)
    Ai = A.astype(np.int64)
    assert np.array_equal(y * 2, (Ai @ B2.T).astype(np.float64))
    assert np.array_equal(ab * 2, (np.abs(Ai) @ np.abs(B2).T).astype(np.float64))


def check_gemm_w4a16_one_hot():
    """One-hot activation rows pick single dequantized weights: with A[m, k] =
    v_m at k = j_m (0 elsewhere), y[m, n] = v_m * dequant(B)[n, j_m], for both
    formats (NVFP4 including the weight tensor scale)."""
    g = workloads.rng(20, 20)
    W = _bf16_f32(workloads.gemm_weight(12, 256, 20))
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        cb, sb, tb = oracle.quantize(W, fmt)
        Wh = oracle.dequantize(cb, sb, fmt, tb).astype(np.float64)
        M = 6
        j = g.integers(0, 256, M)
        v = np.array([1.0, -2.0, 0.5, 3.0, -0.25, 8.0], np.float32)
        A = np.zeros((M, 256), np.float32)
        A[np.arange(M), j] = v
        y, ab = oracle.gemm_w4a16_full(fmt, 256, A, cb, sb, tb)
        ref = v[:, None].astype(np.float64) * Wh[:, j].T
        assert np.allclose(y, ref, rtol=1e-6, atol=0), fmt
        assert np.allclose(ab, np.abs(ref), rtol=1e-6, atol=0), fmt


def check_gemm_w4a16_matches_fp4_gemm():
    """When the activations are exactly representable MXFP4 values (the
    dequantized codes of a random quantized tensor), the weight-only product
    equals the FP4 x FP4 product bit for bit; for NVFP4 (activation values
    rounded to fp32 through their tensor scale) to 1e-6 relative."""
    M, N, K = 4, 9, 512
    for fmt in (oracle.MXFP4, oracle.NVFP4):
        X = _bf16_f32(workloads.gemm_activation(M, K, 21))
        W = _bf16_f32(workloads.gemm_weight(N, K, 21))
        ca, sa, ta = oracle.quantize(X, fmt)
        cb, sb, tb = oracle.quantize(W, fmt)
        Xh = oracle.dequantize(ca, sa, fmt, ta)
        y4, _ = oracle.gemm_full(fmt, K, ca, sa, ta, cb, sb, tb)
        y16, _ = oracle.gemm_w4a16_full(fmt, K, Xh, cb, sb, tb)
        if fmt == oracle.MXFP4:
            assert np.array_equal(y16, y4)
        else:
            assert np.allclose(y16, y4, rtol=1e-6, atol=1e-6 * np.abs(y4).max())


def check_sizes():
    """Bits per element: 4.25 (MXFP4) and 4.5 (NVFP4) from codes plus scales."""
    x = np.ones((4, 256), np.float32)
    for fmt, key in ((oracle.MXFP4, "mxfp4"), (oracle.NVFP4, "nvfp4")):
        c, s, _ = oracle.quantize(x, fmt)
        bits = 8 * (c.nbytes + s.nbytes) / x.size
        assert bits == FMT[key]["bits_per_element"]
        assert 8 * (c.nbytes + s.nbytes) / (x.size / FMT[key]["block"]) == FMT[key]["bits_per_block"]



def check_tiled_code_layout():
    """The tiled code layout at positions worked out by hand from its
    definition (8 KB tiles of 128 rows x 64 bytes; a panel's tiles along the
    row, then the next panel), for a 256 x 512 matrix (256 bytes per row, four
    tiles per panel), and that it only moves bytes."""
    rows, row_bytes = 256, 256
    expected = {(0, 0): 0, (1, 0): 64, (0, 63): 63, (0, 64): 8192, (127, 63): 8191,
                (0, 255): 3 * 8192 + 63, (128, 0): 4 * 8192, (130, 100): 5 * 8192 + 2 * 64 + 36,
                (255, 255): 65535}
    for (r, b), pos in expected.items():
        src = np.zeros((rows, row_bytes), np.uint8)
        src[r, b] = 0xA5
        t = oracle.tile_codes(src)
        assert t.size == rows * row_bytes
        assert np.flatnonzero(t).tolist() == [pos], ((r, b), np.flatnonzero(t)[:4], pos)
    g = np.random.default_rng(3)
    src = g.integers(0, 256, (384, 192), dtype=np.uint8)
    t = oracle.tile_codes(src)
    assert np.array_equal(np.sort(t), np.sort(src.ravel()))
    # a one-panel, one-tile matrix is unchanged
    one = g.integers(0, 256, (128, 64), dtype=np.uint8)
    assert np.array_equal(oracle.tile_codes(one), one.ravel())
    for bad in ((64, 64), (128, 32)):
        try:
            oracle.tile_codes(np.zeros(bad, np.uint8))
        except ValueError:
            continue
        raise AssertionError("tile_codes accepted %r" % (bad,))


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]

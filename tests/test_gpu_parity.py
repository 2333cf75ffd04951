"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Non-rotated codes, scales and tensor scales must match bit for bit; rotated
codes within the 1e-4 adjacent-mismatch budget; dequantized values exactly
(fp32) or to the bf16 rounding of the oracle's fp32; error sums to 1e-9
relative; GEMMs within |y - y_ref| <= 1e-5 (|A||B|) (bf16 output: plus half a
bf16 ulp).  Full-size workloads run in the same launch configuration as the
benchmark; big GEMMs are checked on sampled rows and entries.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import oracle
import workloads
from gpu_common import (assert_rotated_codes_close, assert_rotated_int4_close, assert_search_close,
                        codes_np, gemm_tolerance_ok, rowmajor_scales_np, say, to_dev_bf16, to_dev_f32,
                        to_dev_u8)

pytestmark = pytest.mark.gpu

FMTS = [fp4.FMT_MXFP4, fp4.FMT_NVFP4]
FNAME = {fp4.FMT_MXFP4: "mxfp4", fp4.FMT_NVFP4: "nvfp4", fp4.FMT_MXINT4: "mxint4",
         fp4.FMT_NVINT4: "nvint4"}
INT4 = [fp4.FMT_MXINT4, fp4.FMT_NVINT4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _inputs(name):
    """(label, host fp32 view, device tensor)."""
    if name == "cfg1":
        x = workloads.cfg1_tensor(0)
        return x, to_dev_f32(x)
    if name in ("cfg2_gauss", "cfg2_laplace"):
        b = workloads.cfg2_tensor(name.split("_")[1], 0)
    elif name == "cfg3":
        b = workloads.cfg3_tensor(0)
    elif name == "ragged":
        b = workloads.cfg2_tensor("laplace", 9, rows=37, cols=4128)
    elif name == "tiny_rows":
        b = workloads.cfg2_tensor("gauss", 10, rows=3, cols=96)
    elif name == "tiny_scale":
        # amax near 2^-113: NVFP4 tensor scale near 2^-125 (below 2^-100)
        g = workloads.bf16_bits_to_f32(workloads.cfg2_tensor("gauss", 13, rows=64, cols=1024))
        b = workloads.to_bf16_bits((g * np.float32(2.0 ** -110)).astype(np.float32))
    else:
        raise KeyError(name)
    return workloads.bf16_bits_to_f32(b), to_dev_bf16(b)


NONROT_CASES = ["cfg1", "cfg2_gauss", "cfg2_laplace", "cfg3", "ragged", "tiny_rows", "tiny_scale"]


def _prefill(q):
    q.codes.fill_(0xAA)
    q.scales.fill_(0xAA)
    return q


@pytest.mark.parametrize("case", NONROT_CASES)
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_quantize_bit_exact(case, fmt):
    say("quantize bit-exact", case, FNAME[fmt])
    xh, xd = _inputs(case)
    if fmt == fp4.FMT_NVFP4 and case == "cfg1":
        pass
    layouts = [fp4.SCALES_ROWMAJOR, fp4.SCALES_GEMM] if fmt == fp4.FMT_MXFP4 else [fp4.SCALES_ROWMAJOR]
    rc, rs, rts = oracle.quantize(xh, fmt)
    for lay in layouts:
        q = fp4.quantize(xd, fmt, scale_layout=lay)
        q2 = _prefill(fp4.quantize(xd, fmt, scale_layout=lay))
        fp4.quantize(xd, fmt, scale_layout=lay, out=q2)
        torch.cuda.synchronize()
        gc = codes_np(q)
        gs = rowmajor_scales_np(q)
        assert np.array_equal(gc, rc), (case, lay, np.argwhere(gc != rc)[:5])
        assert np.array_equal(gs, rs), (case, lay, np.argwhere(gs != rs)[:5])
        if fmt == fp4.FMT_NVFP4:
            assert q.global_scale.item() == float(rts), (q.global_scale.item(), rts)
        # deterministic and independent of the previous buffer contents
        assert np.array_equal(codes_np(q2), gc) and np.array_equal(rowmajor_scales_np(q2), gs)


@pytest.mark.parametrize("case", ["cfg2_laplace", "ragged"])
def test_nvfp4_given_global_scale(case):
    say("nvfp4 given ts", case)
    xh, xd = _inputs(case)
    ts = np.float32(0.013)
    rc, rs, _ = oracle.quantize(xh, oracle.NVFP4, ts=ts)
    q = fp4.quantize(xd, fp4.FMT_NVFP4, global_scale=torch.tensor([ts], device="cuda"))
    torch.cuda.synchronize()
    assert q.global_scale.item() == float(ts)
    assert np.array_equal(codes_np(q), rc)
    assert np.array_equal(rowmajor_scales_np(q), rs)


@pytest.mark.parametrize("case", ["cfg2_gauss", "cfg2_laplace", "cfg3", "ragged", "tiny_scale"])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_quantize_rotated(case, fmt):
    say("quantize rotated", case, FNAME[fmt])
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=True)
    lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXFP4 else fp4.SCALES_ROWMAJOR
    q = fp4.quantize(xd, fmt, rotate=True, scale_layout=lay)
    torch.cuda.synchronize()
    if fmt == fp4.FMT_NVFP4:
        g = np.float32(q.global_scale.item())
        assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (g, rts)
    assert_rotated_codes_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)


@pytest.mark.parametrize("case", NONROT_CASES)
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_quantize_int4_bit_exact(case, fmt):
    """MXINT4 / NVINT4, non-rotated: codes, scale codes and the tensor scale bit
    for bit, in every scale layout."""
    say("quantize int4", case, FNAME[fmt])
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize(xh, fmt)
    lays = [fp4.SCALES_GEMM, fp4.SCALES_ROWMAJOR] if fmt == fp4.FMT_MXINT4 else [fp4.SCALES_ROWMAJOR]
    for lay in lays:
        q = _prefill(fp4.quantize(xd, fmt, scale_layout=lay))
        q = fp4.quantize(xd, fmt, scale_layout=lay, out=q)
        torch.cuda.synchronize()
        gc, gs = codes_np(q), rowmajor_scales_np(q)
        assert np.array_equal(gs, rs), (case, lay)
        bad = np.nonzero(gc != rc)
        assert bad[0].size == 0, (case, lay, bad[0][:4], bad[1][:4], gc[bad][:4], rc[bad][:4])
        if fmt == fp4.FMT_NVINT4:
            assert q.global_scale.item() == float(rts)


@pytest.mark.parametrize("case", ["cfg2_laplace", "ragged"])
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_quantize_int4_rotated(case, fmt):
    say("quantize int4 rotated", case, FNAME[fmt])
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=True)
    lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXINT4 else fp4.SCALES_ROWMAJOR
    q = fp4.quantize(xd, fmt, rotate=True, scale_layout=lay)
    torch.cuda.synchronize()
    if fmt == fp4.FMT_NVINT4:
        g = np.float32(q.global_scale.item())
        assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (g, rts)
    assert_rotated_int4_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)


@pytest.mark.parametrize("case", ["cfg1", "cfg2_laplace", "ragged"])
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
@pytest.mark.parametrize("rot", [False, True], ids=["plain", "rot"])
def test_int4_dequantize_and_error_sums(case, fmt, rot):
    """Dequantized INT4 values (of the GPU's own codes) exactly as the oracle
    decodes them; error sums against the oracle's on the same values."""
    say("int4 dequantize", case, FNAME[fmt], rot)
    xh, xd = _inputs(case)
    lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXINT4 else fp4.SCALES_ROWMAJOR
    q = fp4.quantize(xd, fmt, rotate=rot, scale_layout=lay)
    torch.cuda.synchronize()
    gc, gs = codes_np(q), rowmajor_scales_np(q)
    ts = np.float32(q.global_scale.item()) if fmt == fp4.FMT_NVINT4 else np.float32(0)
    ref = oracle.dequantize(gc, gs, fmt, ts)
    y = fp4.dequantize(q).cpu().numpy()
    assert np.array_equal(y, ref)
    yb = fp4.dequantize(q, dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, workloads.bf16_bits_to_f32(workloads.to_bf16_bits(ref)))
    ref_o = oracle.dequantize(gc, gs, fmt, ts, inverse_rotate=rot)
    yo = fp4.dequantize(q, inverse_rotate=rot).cpu().numpy()
    G = fp4.BLOCK[fmt]
    if rot:
        blk = np.abs(ref).reshape(ref.shape[0], -1, G).sum(-1)
        atol = np.repeat(blk, G, axis=1) * 5 * 2.0 ** -24
        assert np.all(np.abs(yo - ref_o) <= atol)
    else:
        assert np.array_equal(yo, ref_o)
    sums = fp4.error_sums(xd, q).cpu().numpy()
    ref_sums = oracle.error_sums(xh, ref_o)
    np.testing.assert_allclose(sums, ref_sums, rtol=1e-9 if not rot else 1e-5)
    say("  nmse %.6e" % (sums[0] / sums[1]))


RULES = [(fp4.FMT_MXFP4, fp4.SCALE_MSE), (fp4.FMT_NVFP4, fp4.SCALE_MSE),
         (fp4.FMT_NVFP4, fp4.SCALE_FOUR_OVER_SIX)]
RULE_IDS = ["mxfp4-mse", "nvfp4-mse", "nvfp4-4over6"]


@pytest.mark.parametrize("case", ["cfg1", "cfg2_gauss", "cfg2_laplace", "ragged", "tiny_rows",
                                  "tiny_scale"])
@pytest.mark.parametrize("fmt,rule", RULES, ids=RULE_IDS)
def test_quantize_scale_search_bit_exact(case, fmt, rule):
    """Searching block-scale rules, non-rotated: codes, scale codes and the
    NVFP4 tensor scale bit for bit (the error sums that decide are fp32 in a
    fixed order on both sides)."""
    say("quantize scale search", case, FNAME[fmt], rule)
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize(xh, fmt, rule=rule)
    lays = [fp4.SCALES_GEMM, fp4.SCALES_ROWMAJOR] if fmt == fp4.FMT_MXFP4 else [fp4.SCALES_ROWMAJOR]
    for lay in lays:
        q = _prefill(fp4.quantize(xd, fmt, scale_layout=lay, rule=rule))
        q = fp4.quantize(xd, fmt, scale_layout=lay, rule=rule, out=q)
        torch.cuda.synchronize()
        gc, gs = codes_np(q), rowmajor_scales_np(q)
        bad = np.nonzero(gs != rs)
        assert bad[0].size == 0, (case, lay, bad[0][:4], bad[1][:4], gs[bad][:4], rs[bad][:4])
        assert np.array_equal(gc, rc), (case, lay)
        if fmt == fp4.FMT_NVFP4:
            assert q.global_scale.item() == float(rts)


@pytest.mark.parametrize("case", ["cfg2_laplace", "ragged"])
@pytest.mark.parametrize("fmt,rule", RULES, ids=RULE_IDS)
def test_quantize_scale_search_rotated(case, fmt, rule):
    say("quantize scale search rotated", case, FNAME[fmt], rule)
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=True, rule=rule)
    lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXFP4 else fp4.SCALES_ROWMAJOR
    q = fp4.quantize(xd, fmt, rotate=True, scale_layout=lay, rule=rule)
    torch.cuda.synchronize()
    ts = rts
    if fmt == fp4.FMT_NVFP4:
        g = np.float32(q.global_scale.item())
        assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (g, rts)
        ts = g
        if g != rts:   # the tensor scales differ by an ulp: compare against the oracle at the GPU's
            rc, rs, _ = oracle.quantize(xh, fmt, rotate=True, ts=g, rule=rule)
    y = oracle.rotate(xh, fp4.BLOCK[fmt])
    assert_search_close(codes_np(q), rowmajor_scales_np(q), rc, rs, fmt, ts, y, what=case)


def test_scale_search_lowers_the_error():
    """On the same tensor the searching rules give a smaller reconstruction
    error than absmax (GPU error sums), and rotation plus MSE scales brings
    NVFP4 below its absmax error ("MR-GPTQ-NVFP4": an MSE-optimised grid on
    rotated weights)."""
    xh, xd = _inputs("cfg2_laplace")
    res = {}
    for fmt, rule in [(fp4.FMT_MXFP4, fp4.SCALE_ABSMAX)] + RULES[:1] + [
            (fp4.FMT_NVFP4, fp4.SCALE_ABSMAX)] + RULES[1:]:
        for rot in (False, True):
            q = fp4.quantize(xd, fmt, rotate=rot, rule=rule)
            s = fp4.error_sums(xd, q).cpu().numpy()
            res[(fmt, rule, rot)] = s[0] / s[1]
    say("  nmse " + " ".join("%s/%d/%s=%.5f" % (FNAME[f], r, "rot" if o else "plain", v)
                              for (f, r, o), v in res.items()))
    for rot in (False, True):
        assert res[(fp4.FMT_MXFP4, fp4.SCALE_MSE, rot)] < res[(fp4.FMT_MXFP4, fp4.SCALE_ABSMAX, rot)]
        assert res[(fp4.FMT_NVFP4, fp4.SCALE_MSE, rot)] < res[(fp4.FMT_NVFP4, fp4.SCALE_FOUR_OVER_SIX, rot)]
        assert res[(fp4.FMT_NVFP4, fp4.SCALE_FOUR_OVER_SIX, rot)] < res[(fp4.FMT_NVFP4, fp4.SCALE_ABSMAX, rot)]
    assert res[(fp4.FMT_NVFP4, fp4.SCALE_MSE, True)] < res[(fp4.FMT_NVFP4, fp4.SCALE_ABSMAX, False)]


@pytest.mark.parametrize("case", ["cfg1", "cfg2_laplace", "ragged"])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
@pytest.mark.parametrize("rot", [False, True], ids=["plain", "rot"])
def test_dequantize_and_error_sums(case, fmt, rot):
    say("dequantize", case, FNAME[fmt], rot)
    xh, xd = _inputs(case)
    lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXFP4 else fp4.SCALES_ROWMAJOR
    q = fp4.quantize(xd, fmt, rotate=rot, scale_layout=lay)
    torch.cuda.synchronize()
    # the oracle dequantizes the GPU's codes only after they were shown equal
    # to its own (non-rotated); for rotated inputs it dequantizes its own codes
    # and the comparison runs on the blocks whose codes agree.
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=rot)
    gc, gs = codes_np(q), rowmajor_scales_np(q)
    ref_rot = oracle.dequantize(rc, rs, fmt, rts)
    ref_orig = oracle.dequantize(rc, rs, fmt, rts, inverse_rotate=True) if rot else ref_rot
    y = fp4.dequantize(q).cpu().numpy()
    yb = fp4.dequantize(q, dtype=torch.bfloat16).float().cpu().numpy()
    yo = fp4.dequantize(q, inverse_rotate=True).cpu().numpy()
    sums = fp4.error_sums(xd, q).cpu().numpy()
    torch.cuda.synchronize()
    G = fp4.BLOCK[fmt]
    same = np.repeat((gs == rs) & (gc.reshape(gc.shape[0], -1, G // 2) == rc.reshape(rc.shape[0], -1, G // 2)).all(-1),
                     G, axis=1)
    if not rot:
        assert same.all()
    assert same.mean() > 0.99
    assert np.array_equal(y[same], ref_rot[same])
    ref_b = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(ref_rot))
    assert np.array_equal(yb[same], ref_b[same])
    if rot and fmt == fp4.FMT_NVFP4:
        # the fp32 butterfly over 16 values with 24-bit significands rounds at
        # each of its 4 stages: error <= 4 * 2^-24 * sum|x^| of the block
        blk = np.abs(ref_rot).reshape(ref_rot.shape[0], -1, G).sum(-1)
        atol = np.repeat(blk, G, axis=1) * 4 * 2.0 ** -24
        assert np.all(np.abs(yo[same] - ref_orig[same]) <= atol[same])
    else:
        assert np.allclose(yo[same], ref_orig[same], rtol=3e-7, atol=0)
    ref_sums = oracle.error_sums(xh, ref_orig)
    tol = 1e-9 if not rot else 1e-4
    np.testing.assert_allclose(sums, ref_sums, rtol=tol)
    # NMSE is the same whichever side computes it
    say("  nmse gpu %.6e oracle %.6e" % (sums[0] / sums[1], ref_sums[0] / ref_sums[1]))


def test_edge_cases():
    say("edge cases")
    # all zeros
    z = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    qm = fp4.quantize(z, fp4.FMT_MXFP4)
    qn = fp4.quantize(z, fp4.FMT_NVFP4)
    torch.cuda.synchronize()
    assert np.all(codes_np(qm) == 0) and np.all(rowmajor_scales_np(qm) == 0)
    assert np.all(codes_np(qn) == 0) and np.all(rowmajor_scales_np(qn) == 0)
    assert qn.global_scale.item() == 0.0
    # tiny, huge, negative zero and saturating values, fp32 input
    vals = np.array([2.0 ** -130, -2.0 ** -140, 1e30, -3e29, -0.0, 0.0, 6.5, -1e-38] * 8, np.float32)
    x = np.stack([vals, vals[::-1], vals * 1e-8, np.roll(vals, 3)]).astype(np.float32)
    xd = to_dev_f32(x)
    for fmt in FMTS:
        for rot in (False, True):
            q = fp4.quantize(xd, fmt, rotate=rot)
            torch.cuda.synchronize()
            rc, rs, rts = oracle.quantize(x, fmt, rotate=rot)
            if not rot:
                assert np.array_equal(codes_np(q), rc), (fmt, rot)
                assert np.array_equal(rowmajor_scales_np(q), rs), (fmt, rot)
                if fmt == fp4.FMT_NVFP4:
                    assert q.global_scale.item() == float(rts)
            else:
                # fp32 butterfly sums of 1e30-sized values round: adjacent codes only
                assert_rotated_codes_close(codes_np(q), rc, rowmajor_scales_np(q), rs, budget=0.05,
                                           what="edge rot")
    # a single row of one block
    one = to_dev_bf16(workloads.cfg2_tensor("gauss", 12, rows=1, cols=32))
    q = fp4.quantize(one, fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM)
    torch.cuda.synchronize()
    rc, rs, _ = oracle.quantize(workloads.bf16_bits_to_f32(workloads.cfg2_tensor("gauss", 12, rows=1, cols=32)), oracle.MXFP4)
    assert np.array_equal(codes_np(q), rc) and np.array_equal(rowmajor_scales_np(q), rs)
    # empty tensor: MXFP4 is a no-op, NVFP4 writes ts = 0
    e = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    q = fp4.quantize(e, fp4.FMT_NVFP4)
    torch.cuda.synchronize()
    assert q.global_scale.item() == 0.0
    fp4.quantize(e, fp4.FMT_MXFP4)


def test_leading_dimension():
    say("leading dimension")
    b = workloads.cfg2_tensor("laplace", 13, rows=40, cols=320)
    full = to_dev_bf16(b)
    view = full[:, :256]
    xh = workloads.bf16_bits_to_f32(b)[:, :256]
    for fmt in FMTS:
        q = fp4.quantize(view, fmt)
        torch.cuda.synchronize()
        rc, rs, rts = oracle.quantize(np.ascontiguousarray(xh), fmt)
        assert np.array_equal(codes_np(q), rc) and np.array_equal(rowmajor_scales_np(q), rs)


def test_scales_to_gemm_layout():
    say("scale relayout")
    for rows, cols in [(37, 4128), (64, 256), (1, 32), (300, 1024)]:
        rm = workloads.random_scales(rows, cols // 32, 0, 254, seed=rows)
        out = fp4.scales_to_gemm_layout(to_dev_u8(rm), rows, cols)
        torch.cuda.synchronize()
        raw = out.cpu().numpy()
        cfg = fp4.qconfig(fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM)
        size = fp4.fp4_scales_bytes(cfg, rows, cols)
        seen = np.zeros(size, bool)
        for r in range(rows):
            for kb in range(cols // 32):
                o = fp4.fp4_scale_offset(cfg, rows, cols, r, kb)
                assert raw[o] == rm[r, kb]
                seen[o] = True
        assert np.all(raw[:size][~seen] == 127)


# ------------------------------------------------------------------- GEMM
def _rand_operands(fmt, M, N, K, seed):
    """Seeded random packed codes and scale bytes (the GEMM's input domain)."""
    G = fp4.BLOCK[fmt]
    ac = workloads.random_codes(M, K, seed, stream=21)
    bc = workloads.random_codes(N, K, seed, stream=22)
    if fmt in fp4.MX_FORMATS:
        asc = workloads.random_scales(M, K // G, 120, 130, seed, stream=23)
        bsc = workloads.random_scales(N, K // G, 118, 124, seed, stream=24)
        ags = bgs = np.float32(0)
    else:
        asc = workloads.random_scales(M, K // G, 0x20, 0x7E, seed, stream=23)
        bsc = workloads.random_scales(N, K // G, 0x10, 0x7E, seed, stream=24)
        ags, bgs = np.float32(0.0371), np.float32(1.7e-5)
    return ac, asc, ags, bc, bsc, bgs


def _device_operand(codes, scales_rm, gs, fmt, rows, K):
    c = to_dev_u8(codes.reshape(-1))
    if fmt in fp4.MX_FORMATS:
        s = fp4.scales_to_gemm_layout(to_dev_u8(scales_rm.reshape(-1)), rows, K, fmt)
    else:
        s = to_dev_u8(scales_rm.reshape(-1))
    g = torch.tensor([float(gs)], dtype=torch.float32, device="cuda")
    cfg = fp4.qconfig(fmt, scale_layout=fp4.SCALES_GEMM)
    return fp4.Quantized(c, s, g, cfg, rows, K)


def _extreme_operands(fmt, M, N, K, seed):
    """Random codes with scales at the ends of their formats' ranges: E8M0
    codes 0/1 against 253/254 (paired so every product of scales is finite,
    ordinary codes on every fourth block), or subnormal and zero E4M3 codes
    on every other block."""
    G = fp4.BLOCK[fmt]
    ac = workloads.random_codes(M, K, seed, stream=31)
    bc = workloads.random_codes(N, K, seed, stream=32)
    mx = fmt in fp4.MX_FORMATS
    # MXINT4 expands n * 2^(c - 127) to bf16, whose largest finite value is
    # just below 2^128: -8 * 2^125 (code 252) overflows it.  The quantizer
    # writes neither the element -8 nor codes above 252 (the largest bf16 input
    # gives 252 with elements in -7 .. 7), so the extreme codes here stop at 251.
    big = (250, 251) if fmt == fp4.FMT_MXINT4 else (253, 254)
    asc = workloads.extreme_scales(M, K // G, "a", mx, seed, stream=33, big_codes=big)
    bsc = workloads.extreme_scales(N, K // G, "b", mx, seed, stream=34, big_codes=big)
    ags, bgs = (np.float32(0), np.float32(0)) if mx else (np.float32(3.5e3), np.float32(2.25e2))
    return ac, asc, ags, bc, bsc, bgs


def _check_gemm(fmt, M, N, K, seed, out_dtype, nrows=8, nent=256, operands=None):
    """GEMM against the oracle on every column of `nrows` random rows (plus
    the first and last row) and `nent` random entries."""
    say("gemm", FNAME[fmt], M, N, K, out_dtype, "extreme scales" if operands else "")
    ac, asc, ags, bc, bsc, bgs = (operands or _rand_operands)(fmt, M, N, K, seed)
    qa = _device_operand(ac, asc, ags, fmt, M, K)
    qb = _device_operand(bc, bsc, bgs, fmt, N, K)
    y = fp4.gemm(qa, qb, out_dtype=out_dtype)
    y2 = fp4.gemm(qa, qb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    g = np.random.default_rng(seed)
    rsel = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, nrows)]))
    rows = np.concatenate([np.repeat(rsel, N), g.integers(0, M, nent)])
    cols = np.concatenate([np.tile(np.arange(N), rsel.size), g.integers(0, N, nent)])
    ref, absref = oracle.gemm_entries(fmt, K, ac, asc, ags, bc, bsc, bgs, rows, cols)
    yh = y.float().cpu().numpy()
    got = yh[rows, cols].astype(np.float64)
    ok = gemm_tolerance_ok(got, ref, absref, out_dtype == torch.bfloat16)
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, (M, N, K, rows[bad[:4]], cols[bad[:4]], got[bad[:4]], ref[bad[:4]])
    assert torch.equal(y, y2)


GEMM_SMALL = [(64, 96, 256), (100, 72, 384), (1, 130, 128), (33, 257, 512), (256, 256, 1024),
              (300, 520, 640), (16, 4096, 4096), (128, 1024, 2048)]


@pytest.mark.parametrize("M,N,K", GEMM_SMALL)
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_small_full_check(fmt, M, N, K):
    _check_gemm(fmt, M, N, K, seed=M + N + K, out_dtype=torch.float32, nrows=min(M, 16), nent=512)


LLAMA8B = [(4096, 4096, 4096), (4096, 6144, 4096), (4096, 14336, 4096), (4096, 4096, 14336)]


OUT_DT = [torch.float32, torch.bfloat16]
OUT_IDS = ["f32out", "bf16out"]


@pytest.mark.parametrize("out_dtype", OUT_DT, ids=OUT_IDS)
@pytest.mark.parametrize("M,N,K", LLAMA8B, ids=["qkvo", "kv6144", "up", "down"])
def test_gemm_mx_llama8b_shapes(M, N, K, out_dtype):
    """Llama-3-8B linears at M = 4096 in the benchmark's launch configuration:
    fp32 output against the bare 1e-5 (|A||B|) bound, bf16 output with its
    half-ulp allowance; every column of 8 random rows plus 256 entries."""
    _check_gemm(fp4.FMT_MXFP4, M, N, K, seed=7, out_dtype=out_dtype,
                nrows=8 if out_dtype == torch.float32 else 2)


LLAMA70B = [(m, n, k) for m in (1, 16, 128, 8192) for (k, n) in ((8192, 28672), (28672, 8192))]


@pytest.mark.parametrize("out_dtype", OUT_DT, ids=OUT_IDS)
@pytest.mark.parametrize("M,N,K", LLAMA70B, ids=["%dx%dx%d" % s for s in LLAMA70B])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_llama70b_mlp_shapes(fmt, M, N, K, out_dtype):
    """Every column of 8 random rows and 256 entries with fp32 output (the bare
    bound); the bf16 output of the same call on 2 rows and 256 entries."""
    _check_gemm(fmt, M, N, K, seed=11, out_dtype=out_dtype,
                nrows=8 if out_dtype == torch.float32 else 2)


# Shapes that take the 256 x 256 tile plan (at least 256 such tiles) with
# ragged M and N, a K with a last 128-K stage (K % 256 == 128), and a split-K
# slice with an odd number of stages; the 256-K ring with 1, 2, 3 and 5 stages
# (its first and last stages differ: stale reads and a re-load of the last
# stage past the end).
PLAN_EDGES = [(4000, 4100, 4096), (4000, 4100, 4224), (64, 1024, 1152), (4000, 4100, 1024),
              (4096, 4096, 256), (4000, 4100, 512), (4000, 4100, 768), (4096, 4096, 1280),
              # unsplit 128 x 128 tiles above 128 rows (the 256-K kernel, eight waves
              # of 64 x 32): ragged, three stages, and full-size medium shapes
              (300, 1000, 768), (2048, 4096, 4096), (520, 14336, 4096), (129, 2000, 256),
              # shapes the split-K plan used to take (few tiles, long K)
              (256, 1024, 8192), (2048, 1000, 2048)]


@pytest.mark.parametrize("out_dtype", OUT_DT, ids=OUT_IDS)
@pytest.mark.parametrize("M,N,K", PLAN_EDGES, ids=["%dx%dx%d" % s for s in PLAN_EDGES])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_tile_plan_edges(fmt, M, N, K, out_dtype):
    _check_gemm(fmt, M, N, K, seed=M + K, out_dtype=out_dtype)


# Wide decode shapes (M <= 32) with ragged last column tiles, every row checked.
WIDE_DECODE = [(1, 28672, 1024), (7, 26000, 1024), (32, 25088, 512), (16, 32000, 768)]


@pytest.mark.parametrize("out_dtype", OUT_DT, ids=OUT_IDS)
@pytest.mark.parametrize("M,N,K", WIDE_DECODE, ids=["%dx%dx%d" % s for s in WIDE_DECODE])
def test_gemm_wide_decode_ragged(M, N, K, out_dtype):
    _check_gemm(fp4.FMT_MXFP4, M, N, K, seed=N + K, out_dtype=out_dtype, nrows=M)


EXTREME = [(256, 512, 1024), (16, 4096, 4096), (4000, 4100, 4096), (128, 4096, 8192)]


@pytest.mark.parametrize("M,N,K", EXTREME, ids=["%dx%dx%d" % s for s in EXTREME])
@pytest.mark.parametrize("fmt", FMTS + INT4, ids=["mxfp4", "nvfp4", "mxint4", "nvint4"])
def test_gemm_extreme_scales(fmt, M, N, K):
    """E8M0 codes 0, 1, 253, 254 (products of scales from 2^-1 to 2^1 and
    ordinary ones) and E4M3 subnormal / zero block scales reach the MFMA
    paths: fp32 output against the bare bound."""
    _check_gemm(fmt, M, N, K, seed=K + N, out_dtype=torch.float32, operands=_extreme_operands)


@pytest.mark.parametrize("fmt", FMTS + INT4, ids=["mxfp4", "nvfp4", "mxint4", "nvint4"])
def test_gemm_split_k_workspace_reuse(fmt):
    """One workspace serves split-K calls of different shapes in turn (any
    contents on entry), and the results are repeatable bit for bit and within
    the bound."""
    ws = fp4.gemm_workspace(1 << 26, "cuda")
    for (M, N, K) in ((16, 4096, 8192), (1, 2048, 28672), (128, 1024, 4096), (16, 4096, 8192)):
        assert fp4.fp4_gemm_workspace_bytes(fmt, M, N, K) > 0
        ac, asc, ags, bc, bsc, bgs = _rand_operands(fmt, M, N, K, seed=M + K)
        qa = _device_operand(ac, asc, ags, fmt, M, K)
        qb = _device_operand(bc, bsc, bgs, fmt, N, K)
        y1 = fp4.gemm(qa, qb, out_dtype=torch.float32, workspace=ws)
        y2 = fp4.gemm(qa, qb, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        rows = np.repeat(np.arange(M), 64)
        cols = np.tile(np.arange(0, N, N // 64), M)
        ref, absref = oracle.gemm_entries(fmt, K, ac, asc, ags, bc, bsc, bgs, rows, cols)
        got = y1.cpu().numpy()[rows, cols].astype(np.float64)
        assert np.all(gemm_tolerance_ok(got, ref, absref, False)), (M, N, K)


@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_quantize_then_gemm_end_to_end(fmt):
    """bf16 activations and weights quantized on the GPU (non-rotated, hence
    bit-identical to the oracle's codes), multiplied on the GPU, against the
    oracle's quantize + product."""
    M, N, K = 256, 384, 1024
    say("end to end", FNAME[fmt])
    xa = workloads.gemm_activation(M, K, seed=3)
    xb = workloads.gemm_weight(N, K, seed=3)
    qa = fp4.quantize(to_dev_bf16(xa), fmt, scale_layout=fp4.SCALES_GEMM)
    qb = fp4.quantize(to_dev_bf16(xb), fmt, scale_layout=fp4.SCALES_GEMM)
    y = fp4.gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ca, sa, ga = oracle.quantize(workloads.bf16_bits_to_f32(xa), fmt)
    cb, sb, gb = oracle.quantize(workloads.bf16_bits_to_f32(xb), fmt)
    assert np.array_equal(codes_np(qa), ca) and np.array_equal(codes_np(qb), cb)
    rows = np.repeat(np.arange(0, M, 7), N)
    cols = np.tile(np.arange(N), np.arange(0, M, 7).size)
    ref, absref = oracle.gemm_entries(fmt, K, ca, sa, ga, cb, sb, gb, rows, cols)
    got = y.cpu().numpy()[rows, cols].astype(np.float64)
    assert np.all(gemm_tolerance_ok(got, ref, absref, False))


# ---------------------------------------------------------------- W4A16


def _check_w4a16(fmt, M, N, K, seed, out_dtype, lda_pad=0, nrows=8, nent=256, split=True):
    say("w4a16", FNAME[fmt], M, N, K, out_dtype, "lda+%d" % lda_pad, "split" if split else "unsplit")
    _, _, _, bc, bsc, bgs = _rand_operands(fmt, M, N, K, seed)
    qb = _device_operand(bc, bsc, bgs, fmt, N, K)
    abits = workloads.gemm_activation(M, K + lda_pad, seed=seed)
    a_full = to_dev_bf16(abits)
    a = a_full[:, :K]
    y = torch.empty(M, N, dtype=out_dtype, device="cuda")
    if split:
        fp4.gemm_w4a16(a, qb, out=y)
    else:
        rc = fp4.fp4_gemm_w4a16(fmt, M, N, K, a.data_ptr(), a.stride(0), qb.codes.data_ptr(),
                                qb.scales.data_ptr(), qb.global_scale.data_ptr(), y.data_ptr(),
                                fp4.DT_F32 if out_dtype == torch.float32 else fp4.DT_BF16, N, None, 0,
                                torch.cuda.current_stream().cuda_stream)
        assert rc == fp4.FP4_OK
    torch.cuda.synchronize()
    g = np.random.default_rng(seed)
    rsel = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, nrows)]))
    rows = np.concatenate([np.repeat(rsel, N), g.integers(0, M, nent)])
    cols = np.concatenate([np.tile(np.arange(N), rsel.size), g.integers(0, N, nent)])
    av = workloads.bf16_bits_to_f32(abits)[:, :K]
    ref, absref = oracle.gemm_w4a16_entries(fmt, K, av, bc, bsc, bgs, rows, cols)
    got = y.float().cpu().numpy()[rows, cols].astype(np.float64)
    ok = gemm_tolerance_ok(got, ref, absref, out_dtype == torch.bfloat16)
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, (M, N, K, rows[bad[:4]], cols[bad[:4]], got[bad[:4]], ref[bad[:4]])
    return y


W4_SMALL = [(1, 64, 256), (7, 96, 512), (16, 300, 768), (33, 520, 1024), (64, 200, 512),
            (100, 256, 256), (128, 384, 1024), (257, 130, 512), (1, 4096, 4096), (16, 1024, 2048)]


@pytest.mark.parametrize("M,N,K", W4_SMALL, ids=["%dx%dx%d" % s for s in W4_SMALL])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_w4a16_small_full_check(fmt, M, N, K):
    _check_w4a16(fmt, M, N, K, seed=M + N + K, out_dtype=torch.float32, nrows=min(M, 16), nent=512)


@pytest.mark.parametrize("M", [16, 48, 100], ids=["rows32", "rows64", "rows128"])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_w4a16_strided_activations_and_unsplit(fmt, M):
    """A row-strided activation view (lda > K) through each row tile (32, 64
    and 128 rows), and the call without a workspace (one pass over K)
    against the oracle and the split result."""
    N, K = 768, 4096
    y1 = _check_w4a16(fmt, M, N, K, seed=5, out_dtype=torch.float32, lda_pad=64, nrows=16)
    y2 = _check_w4a16(fmt, M, N, K, seed=5, out_dtype=torch.float32, lda_pad=64, nrows=16, split=False)
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fmt, M, N, K) > 0
    assert torch.allclose(y1, y2, rtol=0, atol=1e-3 * float(y1.abs().max()))


LLAMA70B_DECODE = [(m, n, k) for m in (1, 16, 128) for (k, n) in ((8192, 28672), (28672, 8192))]


@pytest.mark.parametrize("out_dtype", OUT_DT, ids=OUT_IDS)
@pytest.mark.parametrize("M,N,K", LLAMA70B_DECODE, ids=["%dx%dx%d" % s for s in LLAMA70B_DECODE])
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_w4a16_llama70b_mlp_shapes(fmt, M, N, K, out_dtype):
    _check_w4a16(fmt, M, N, K, seed=13, out_dtype=out_dtype,
                 nrows=8 if out_dtype == torch.float32 else 2)


@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_gemm_w4a16_quantized_weights_end_to_end(fmt):
    """bf16 weights quantized on the GPU (bit-identical to the oracle's codes),
    then the weight-only product against the oracle's."""
    M, N, K = 16, 384, 1024
    say("w4a16 end to end", FNAME[fmt])
    xa = workloads.gemm_activation(M, K, seed=4)
    xb = workloads.gemm_weight(N, K, seed=4)
    qb = fp4.quantize(to_dev_bf16(xb), fmt, scale_layout=fp4.SCALES_GEMM)
    y = fp4.gemm_w4a16(to_dev_bf16(xa), qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cb, sb, gb = oracle.quantize(workloads.bf16_bits_to_f32(xb), fmt)
    assert np.array_equal(codes_np(qb), cb)
    r, c = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, absref = oracle.gemm_w4a16_entries(fmt, K, workloads.bf16_bits_to_f32(xa), cb, sb, gb,
                                            r.reshape(-1), c.reshape(-1))
    got = y.cpu().numpy().reshape(-1).astype(np.float64)
    assert np.all(gemm_tolerance_ok(got, ref, absref, False))


def test_gemm_w4a16_empty_k_writes_zeros():
    say("w4a16 K=0")
    y = torch.full((3, 5), 7.0, dtype=torch.float32, device="cuda")
    a = torch.zeros(3, 0, dtype=torch.bfloat16, device="cuda")
    rc = fp4.fp4_gemm_w4a16(fp4.FMT_NVFP4, 3, 5, 0, a.data_ptr(), 0, None, None, None, y.data_ptr(),
                            fp4.DT_F32, 5, None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == fp4.FP4_OK
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


# ------------------------------------------------------ INT4 element GEMMs
INT4_GEMM = [(64, 96, 256), (1, 130, 512), (33, 257, 512), (256, 256, 1024), (300, 520, 768),
             (16, 4096, 4096), (128, 1024, 2048)]


@pytest.mark.parametrize("M,N,K", INT4_GEMM, ids=["%dx%dx%d" % s for s in INT4_GEMM])
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_gemm_int4_small_full_check(fmt, M, N, K):
    """MXINT4 / NVINT4 operands (every nibble, -8 included) against the
    oracle's double-precision product."""
    _check_gemm(fmt, M, N, K, seed=M + N + K, out_dtype=torch.float32, nrows=min(M, 16), nent=512)


@pytest.mark.parametrize("M,N,K", [(8192, 28672, 8192), (16, 8192, 28672)], ids=["8192x28672x8192", "16x8192x28672"])
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_gemm_int4_llama70b_shapes(fmt, M, N, K):
    _check_gemm(fmt, M, N, K, seed=17, out_dtype=torch.float32)


@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_int4_quantize_then_gemm_end_to_end(fmt):
    M, N, K = 256, 384, 1024
    say("int4 end to end", FNAME[fmt])
    xa = workloads.gemm_activation(M, K, seed=5)
    xb = workloads.gemm_weight(N, K, seed=5)
    qa = fp4.quantize(to_dev_bf16(xa), fmt, scale_layout=fp4.SCALES_GEMM)
    qb = fp4.quantize(to_dev_bf16(xb), fmt, scale_layout=fp4.SCALES_GEMM)
    y = fp4.gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ca, sa, ga = oracle.quantize(workloads.bf16_bits_to_f32(xa), fmt)
    cb, sb, gb = oracle.quantize(workloads.bf16_bits_to_f32(xb), fmt)
    assert np.array_equal(codes_np(qa), ca) and np.array_equal(codes_np(qb), cb)
    rows = np.repeat(np.arange(0, M, 7), N)
    cols = np.tile(np.arange(N), np.arange(0, M, 7).size)
    ref, absref = oracle.gemm_entries(fmt, K, ca, sa, ga, cb, sb, gb, rows, cols)
    got = y.cpu().numpy()[rows, cols].astype(np.float64)
    assert np.all(gemm_tolerance_ok(got, ref, absref, False))


W4_INT4 = [(1, 64, 256), (16, 300, 768), (33, 520, 1024), (65, 384, 768), (128, 1024, 2048),
           (1, 8192, 28672)]


@pytest.mark.parametrize("M,N,K", W4_INT4, ids=["%dx%dx%d" % s for s in W4_INT4])
@pytest.mark.parametrize("fmt", INT4, ids=["mxint4", "nvint4"])
def test_gemm_w4a16_int4_weights(fmt, M, N, K):
    _check_w4a16(fmt, M, N, K, seed=M + N + K, out_dtype=torch.float32, nrows=min(M, 8), nent=256)


# ------------------------------------------- rotation and rounding variants
MASK = 0x0123456789ABCDEF0FEDCBA987654321
ROTS = [(fp4.FMT_MXFP4, 32, MASK), (fp4.FMT_MXFP4, 64, 0), (fp4.FMT_MXFP4, 64, MASK),
        (fp4.FMT_MXFP4, 128, 0), (fp4.FMT_MXFP4, 128, MASK), (fp4.FMT_NVFP4, 16, MASK),
        (fp4.FMT_MXINT4, 128, MASK), (fp4.FMT_NVINT4, 16, MASK)]
ROT_IDS = ["%s-h%d%s" % (FNAME[f], n, "-signed" if m else "") for f, n, m in ROTS]


@pytest.mark.parametrize("case", ["cfg2_laplace", "ragged"])
@pytest.mark.parametrize("fmt,n,mask", ROTS, ids=ROT_IDS)
def test_quantize_rotation_variants(case, fmt, n, mask):
    """Sign-randomised rotations and 64 / 128-point MX rotations (cross-lane
    butterflies): codes within the rotated budget of the oracle's."""
    say("quantize rotation", case, FNAME[fmt], n, hex(mask))
    xh, xd = _inputs(case)
    if xh.shape[1] % n:
        pytest.skip("cols not a multiple of the rotation")
    rc, rs, rts = oracle.quantize_spec(xh, fmt, rot_n=n, signs=mask)
    lay = fp4.SCALES_GEMM if fmt in fp4.MX_FORMATS else fp4.SCALES_ROWMAJOR
    for layout in ([lay, fp4.SCALES_ROWMAJOR] if lay == fp4.SCALES_GEMM else [lay]):
        q = fp4.quantize(xd, fmt, rotate=n, scale_layout=layout, signs=mask)
        torch.cuda.synchronize()
        if fmt not in fp4.MX_FORMATS:
            g = np.float32(q.global_scale.item())
            assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (g, rts)
        if fmt in INT4:
            assert_rotated_int4_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)
        else:
            assert_rotated_codes_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)
    # back to the original domain: inverse rotation of the GPU's codes
    gc, gs = codes_np(q), rowmajor_scales_np(q)
    ts = np.float32(q.global_scale.item()) if fmt not in fp4.MX_FORMATS else np.float32(0)
    ref = oracle.dequantize_rot(gc, gs, fmt, ts, rot_n=n, signs=mask)
    yo = fp4.dequantize(q, inverse_rotate=True).cpu().numpy()
    grp = np.abs(oracle.dequantize(gc, gs, fmt, ts)).reshape(ref.shape[0], -1, n).sum(-1)
    atol = np.repeat(grp, n, axis=1) * 8 * 2.0 ** -24
    assert np.all(np.abs(yo - ref) <= atol)
    sums = fp4.error_sums(xd, q).cpu().numpy()
    np.testing.assert_allclose(sums, oracle.error_sums(xh, ref), rtol=1e-5)


SR_CASES = ["cfg1", "cfg2_gauss", "ragged", "tiny_rows", "tiny_scale"]


@pytest.mark.parametrize("case", SR_CASES)
@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_quantize_stochastic_rounding_bit_exact(case, fmt):
    """Stochastic rounding, non-rotated: the Philox4x32-10 stream and every
    rounding decision match the oracle bit for bit."""
    say("quantize stochastic", case, FNAME[fmt])
    xh, xd = _inputs(case)
    seed = (0x12345678, 0x9ABCDEF0)
    rc, rs, rts = oracle.quantize_spec(xh, fmt, rounding=oracle.ROUND_STOCHASTIC, seed=seed)
    lays = [fp4.SCALES_GEMM, fp4.SCALES_ROWMAJOR] if fmt == fp4.FMT_MXFP4 else [fp4.SCALES_ROWMAJOR]
    for lay in lays:
        q = _prefill(fp4.quantize(xd, fmt, scale_layout=lay, rounding=fp4.ROUND_STOCHASTIC, seed=seed))
        q = fp4.quantize(xd, fmt, scale_layout=lay, rounding=fp4.ROUND_STOCHASTIC, seed=seed, out=q)
        torch.cuda.synchronize()
        gc, gs = codes_np(q), rowmajor_scales_np(q)
        assert np.array_equal(gs, rs), (case, lay)
        bad = np.nonzero(gc != rc)
        assert bad[0].size == 0, (case, lay, bad[0][:4], bad[1][:4], gc[bad][:4], rc[bad][:4])


@pytest.mark.parametrize("fmt", FMTS, ids=["mxfp4", "nvfp4"])
def test_quantize_stochastic_rounding_rotated(fmt):
    say("quantize stochastic rotated", FNAME[fmt])
    xh, xd = _inputs("cfg2_laplace")
    seed = (7, 11)
    rc, rs, _ = oracle.quantize_spec(xh, fmt, rot_n=fp4.BLOCK[fmt], signs=MASK,
                                     rounding=oracle.ROUND_STOCHASTIC, seed=seed)
    q = fp4.quantize(xd, fmt, rotate=True, signs=MASK, rounding=fp4.ROUND_STOCHASTIC, seed=seed)
    torch.cuda.synchronize()
    assert_rotated_codes_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what="sr rot")


@pytest.mark.parametrize("case", ["cfg1", "cfg2_gauss", "cfg2_laplace", "ragged", "tiny_rows", "tiny_scale"])
@pytest.mark.parametrize("rnd", [0, 1], ids=["nearest", "stochastic"])
def test_quantize_nvfp4_16x16_blocks(case, rnd):
    """NVFP4 16x16 weight blocks: scale codes, element codes and the tensor scale
    bit for bit (ragged row counts included)."""
    say("quantize nvfp4 16x16", case, rnd)
    xh, xd = _inputs(case)
    rc, rs, rts = oracle.quantize_spec(xh, fp4.FMT_NVFP4, block_rows=16, rounding=rnd, seed=(3, 4))
    q = _prefill(fp4.quantize(xd, fp4.FMT_NVFP4, block_rows=16, rounding=rnd, seed=(3, 4)))
    q = fp4.quantize(xd, fp4.FMT_NVFP4, block_rows=16, rounding=rnd, seed=(3, 4), out=q)
    torch.cuda.synchronize()
    assert q.global_scale.item() == float(rts)
    assert np.array_equal(rowmajor_scales_np(q), rs)
    assert np.array_equal(codes_np(q), rc)

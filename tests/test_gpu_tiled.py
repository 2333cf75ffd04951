"""GPU parity of the tiled code layout (FP4_CODES_TILED for fp4_quantize /
fp4_dequantize / fp4_error_sums, fmt | FP4_GEMM_B_TILED for the GEMMs).

Quantize: the tiled codes are the oracle's tiling of the oracle's row-major
codes, bit for bit (rotated encodings: of the library's row-major codes, whose
arithmetic the row-major parity tests cover), with the same scales and tensor
scale.  Dequantize and the error sums read tiled codes back to identical
values.  GEMM: a product with tiled B is bit-identical to the same product with
row-major B (fp32 output) in every tile plan of every entry point, and the
tiled decode products meet the oracle's tolerance directly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import oracle
import workloads
from gpu_common import codes_np, gemm_tolerance_ok, rowmajor_scales_np, say, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

FNAME = {fp4.FMT_MXFP4: "mxfp4", fp4.FMT_NVFP4: "nvfp4", fp4.FMT_MXINT4: "mxint4",
         fp4.FMT_NVINT4: "nvint4"}
ALL = [fp4.FMT_MXFP4, fp4.FMT_NVFP4, fp4.FMT_MXINT4, fp4.FMT_NVINT4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _tiled_np(q: fp4.Quantized) -> np.ndarray:
    return q.codes[: q.rows * q.cols // 2].cpu().numpy()


def _gemm_scales(fmt):
    return fp4.SCALES_GEMM if fmt in fp4.MX_FORMATS else fp4.SCALES_ROWMAJOR


# (id, fmt, input dtype, quantize() keyword arguments): one case per quantize
# kernel family (row tiles, GEMM-layout MX tiles, fp32 input, rotation groups
# of 4 blocks, NVFP4 two-dimensional blocks, the single pass, the scale
# searches, stochastic rounding, the INT4 elements).
QCASES = [
    ("mx_bf16", fp4.FMT_MXFP4, "bf16", {}),
    ("mx_bf16_gemm_scales", fp4.FMT_MXFP4, "bf16", {"scale_layout": fp4.SCALES_GEMM}),
    ("mx_f32", fp4.FMT_MXFP4, "f32", {}),
    ("mx_mse", fp4.FMT_MXFP4, "bf16", {"rule": fp4.SCALE_MSE}),
    ("mx_sr", fp4.FMT_MXFP4, "bf16", {"rounding": fp4.ROUND_STOCHASTIC, "seed": (7, 9)}),
    ("nv_bf16", fp4.FMT_NVFP4, "bf16", {}),
    ("nv_f32", fp4.FMT_NVFP4, "f32", {}),
    ("nv_2d", fp4.FMT_NVFP4, "bf16", {"block_rows": 16}),
    ("nv_one_pass", fp4.FMT_NVFP4, "bf16", {"one_pass": True}),
    ("nv_four_over_six", fp4.FMT_NVFP4, "bf16", {"rule": fp4.SCALE_FOUR_OVER_SIX}),
    ("mxint4", fp4.FMT_MXINT4, "bf16", {"scale_layout": fp4.SCALES_GEMM}),
    ("nvint4", fp4.FMT_NVINT4, "bf16", {}),
]
ROT_CASES = [
    ("mx_h32", fp4.FMT_MXFP4, {"rotate": True, "scale_layout": fp4.SCALES_GEMM}),
    ("mx_h128_signs", fp4.FMT_MXFP4, {"rotate": 128, "signs": 0x5A5A5A5A}),
    ("nv_h16", fp4.FMT_NVFP4, {"rotate": True}),
    ("nv_h16_one_pass", fp4.FMT_NVFP4, {"rotate": True, "one_pass": True}),
    ("mxint4_h32", fp4.FMT_MXINT4, {"rotate": True}),
    ("nvint4_h16", fp4.FMT_NVINT4, {"rotate": True}),
]


def _input(dt, rows=384, cols=1024, seed=0):
    b = workloads.cfg2_tensor("laplace", seed, rows=rows, cols=cols)
    x = workloads.bf16_bits_to_f32(b)
    return x, (to_dev_bf16(b) if dt == "bf16" else to_dev_f32(x))


@pytest.mark.parametrize("case", QCASES, ids=[c[0] for c in QCASES])
def test_quantize_tiled_codes_match_the_oracle(case):
    name, fmt, dt, kw = case
    say("quantize tiled", name)
    x, xd = _input(dt)
    row = fp4.quantize(xd, fmt, code_layout=fp4.CODES_ROWMAJOR, **kw)
    til = fp4.quantize(xd, fmt, code_layout=fp4.CODES_TILED, **kw)
    torch.cuda.synchronize()
    rc = codes_np(row)
    assert np.array_equal(_tiled_np(til), oracle.tile_codes(rc))
    assert np.array_equal(rowmajor_scales_np(til), rowmajor_scales_np(row))
    assert torch.equal(til.global_scale, row.global_scale)
    if name in ("mx_bf16", "mx_f32", "nv_bf16", "nv_f32", "mxint4", "nvint4"):
        # plain absmax encodings: the oracle's own codes, tiled
        oc, osc, ots = oracle.quantize(x, fmt)
        assert np.array_equal(_tiled_np(til), oracle.tile_codes(oc))
        assert np.array_equal(rowmajor_scales_np(til), osc)


@pytest.mark.parametrize("case", ROT_CASES, ids=[c[0] for c in ROT_CASES])
def test_quantize_tiled_rotated(case):
    name, fmt, kw = case
    say("quantize tiled rotated", name)
    _, xd = _input("bf16", seed=3)
    row = fp4.quantize(xd, fmt, **kw)
    til = fp4.quantize(xd, fmt, code_layout=fp4.CODES_TILED, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(_tiled_np(til), oracle.tile_codes(codes_np(row)))
    assert np.array_equal(rowmajor_scales_np(til), rowmajor_scales_np(row))
    assert torch.equal(til.global_scale, row.global_scale)


def test_quantize_batch_tiled_jobs():
    say("quantize_batch tiled")
    xs = [_input("bf16", rows=256, cols=512, seed=s)[1] for s in range(4)]
    items = [dict(x=xs[0], fmt=fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM),
             dict(x=xs[1], fmt=fp4.FMT_MXFP4, rotate=True, scale_layout=fp4.SCALES_GEMM),
             dict(x=xs[2], fmt=fp4.FMT_NVFP4),
             dict(x=xs[3], fmt=fp4.FMT_NVFP4, rotate=True)]
    row = fp4.quantize_batch(items)
    til = fp4.quantize_batch([dict(it, code_layout=fp4.CODES_TILED) for it in items])
    torch.cuda.synchronize()
    for r, t in zip(row, til):
        assert np.array_equal(_tiled_np(t), oracle.tile_codes(codes_np(r)))
        assert np.array_equal(rowmajor_scales_np(t), rowmajor_scales_np(r))
        assert torch.equal(t.global_scale, r.global_scale)


@pytest.mark.parametrize("fmt", ALL, ids=[FNAME[f] for f in ALL])
def test_dequantize_and_error_sums_read_tiled_codes(fmt):
    say("dequantize tiled", FNAME[fmt])
    _, xd = _input("bf16", seed=5)
    for rot in (False, True):
        row = fp4.quantize(xd, fmt, rotate=rot)
        til = fp4.quantize(xd, fmt, rotate=rot, code_layout=fp4.CODES_TILED)
        for inv in (False, True):
            assert torch.equal(fp4.dequantize(til, inverse_rotate=inv),
                               fp4.dequantize(row, inverse_rotate=inv))
        assert torch.equal(fp4.error_sums(xd, til), fp4.error_sums(xd, row))


def _operands(fmt, M, N, K, seed):
    xa = workloads.gemm_activation(M, K, seed=seed)
    xb = workloads.gemm_weight(N, K, seed=seed)
    sl = _gemm_scales(fmt)
    qa = fp4.quantize(to_dev_bf16(xa), fmt, scale_layout=sl)
    qb = fp4.quantize(to_dev_bf16(xb), fmt, scale_layout=sl)
    qt = fp4.quantize(to_dev_bf16(xb), fmt, scale_layout=sl, code_layout=fp4.CODES_TILED)
    return xa, qa, qb, qt


# Shapes that take each tile plan: decode rows (split-K), 128-row tiles at
# M <= 128 and above, 256 x 256 tiles with K % 256 == 0 and == 128, and the
# NVFP4 path for K % 256 == 128.
GEMM_CASES = [
    (fp4.FMT_MXFP4, 1, 1024, 2048), (fp4.FMT_MXFP4, 16, 1024, 2048), (fp4.FMT_MXFP4, 200, 512, 1024),
    (fp4.FMT_MXFP4, 16, 25088, 1024), (fp4.FMT_MXFP4, 384, 4096, 768),
    (fp4.FMT_MXFP4, 4096, 4096, 512), (fp4.FMT_MXFP4, 4096, 4096, 384), (fp4.FMT_MXFP4, 4000, 4224, 768),
    (fp4.FMT_NVFP4, 16, 1024, 2048), (fp4.FMT_NVFP4, 128, 1024, 2048), (fp4.FMT_NVFP4, 256, 1024, 2048),
    (fp4.FMT_NVFP4, 4096, 4096, 512), (fp4.FMT_NVFP4, 64, 256, 384),
    (fp4.FMT_MXINT4, 16, 1024, 2048), (fp4.FMT_MXINT4, 128, 1024, 2048),
    (fp4.FMT_MXINT4, 4096, 4096, 512),
    (fp4.FMT_NVINT4, 16, 1024, 2048), (fp4.FMT_NVINT4, 256, 1024, 2048),
    (fp4.FMT_NVINT4, 4096, 4096, 512),
]


@pytest.mark.parametrize("fmt,M,N,K", GEMM_CASES,
                         ids=["%s-%dx%dx%d" % (FNAME[c[0]], *c[1:]) for c in GEMM_CASES])
def test_gemm_tiled_b_is_bit_identical(fmt, M, N, K):
    say("gemm tiled B", FNAME[fmt], M, N, K)
    _, qa, qb, qt = _operands(fmt, M, N, K, seed=21)
    y_row = fp4.gemm(qa, qb, out_dtype=torch.float32)
    y_til = fp4.gemm(qa, qt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_til, y_row)
    assert bool(torch.isfinite(y_row).all())
    assert torch.equal(fp4.gemm(qa, qt), fp4.gemm(qa, qb))  # bf16 output kernels
    if fp4.fp4_gemm_workspace_bytes(fmt, M, N, K) > 0:  # the unsplit pass as well
        w0 = torch.empty(0, dtype=torch.uint8, device="cuda")
        u_row = fp4.gemm(qa, qb, out_dtype=torch.float32, workspace=w0)
        u_til = fp4.gemm(qa, qt, out_dtype=torch.float32, workspace=w0)
        assert torch.equal(u_til, u_row)


W4_CASES = [(f, M) for f in ALL for M in (16, 48, 100)]


@pytest.mark.parametrize("fmt,M", W4_CASES, ids=["%s-m%d" % (FNAME[f], M) for f, M in W4_CASES])
def test_gemm_w4a16_tiled_b_is_bit_identical(fmt, M):
    N, K = 768, 4096
    say("w4a16 tiled B", FNAME[fmt], M, N, K)
    xa, _, qb, qt = _operands(fmt, M, N, K, seed=22)
    a = to_dev_bf16(xa)
    for ws in (None, torch.empty(0, dtype=torch.uint8, device="cuda")):
        y_row = fp4.gemm_w4a16(a, qb, out_dtype=torch.float32, workspace=ws)
        y_til = fp4.gemm_w4a16(a, qt, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_til, y_row)


@pytest.mark.parametrize("fmt", ALL, ids=[FNAME[f] for f in ALL])
def test_tiled_decode_gemms_against_the_oracle(fmt):
    """Decode rows with tiled weights against the oracle's entries: FP4 x FP4
    (row-major activations) and the weight-only product."""
    M, N, K = 16, 256, 1024
    say("tiled decode vs oracle", FNAME[fmt])
    xa, qa, _, qt = _operands(fmt, M, N, K, seed=23)
    fa, fb = workloads.bf16_bits_to_f32(xa), workloads.bf16_bits_to_f32(workloads.gemm_weight(N, K, seed=23))
    ca, sa, ga = oracle.quantize(fa, fmt)
    cb, sb, gb = oracle.quantize(fb, fmt)
    r, c = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    r, c = r.reshape(-1), c.reshape(-1)
    y = fp4.gemm(qa, qt, out_dtype=torch.float32)
    ref, absref = oracle.gemm_entries(fmt, K, ca, sa, ga, cb, sb, gb, r, c)
    assert np.all(gemm_tolerance_ok(y.cpu().numpy().reshape(-1).astype(np.float64), ref, absref, False))
    y16 = fp4.gemm_w4a16(to_dev_bf16(xa), qt, out_dtype=torch.float32)
    ref16, abs16 = oracle.gemm_w4a16_entries(fmt, K, fa, cb, sb, gb, r, c)
    assert np.all(gemm_tolerance_ok(y16.cpu().numpy().reshape(-1).astype(np.float64), ref16, abs16, False))


def test_gemm_rejects_tiled_activations():
    _, xd = _input("bf16", rows=128, cols=512)
    qa = fp4.quantize(xd, fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM, code_layout=fp4.CODES_TILED)
    with pytest.raises(ValueError):
        fp4.gemm(qa, qa)
    with pytest.raises(ValueError):
        fp4.codes_view(qa)

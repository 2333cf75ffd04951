"""GPU parity at the edges of the formats, through every bf16 quantize kernel.

Inputs (workloads.edge_tensor) mix 16-element groups of edge kinds: block
maxima below 2^-125 (the E8M0 clamp at 2^-127), bf16 subnormals, +0 / -0,
values up to 3e38 (saturating onto +-6), single non-zero elements, and, for
the NV formats, block maxima far below the tensor maximum (subnormal and zero
E4M3 block scales).  Each is quantized through the separate-call kernels
(row-major and GEMM-layout scales), the single-pass NVFP4 kernel, the
grouped batch kernel and the given-tensor-scale path, and compared with the
oracle: bit for bit without rotation, within the rotated budget with it.
Also: two streams quantizing NVFP4 at once (each with its own workspace), and
the single-pass give-up check on a clean call and on a flagged workspace.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import oracle
import workloads
from gpu_common import (assert_rotated_codes_close, assert_rotated_int4_close, codes_np,
                        rowmajor_scales_np, say, to_dev_bf16)

pytestmark = pytest.mark.gpu

FNAME = {fp4.FMT_MXFP4: "mxfp4", fp4.FMT_NVFP4: "nvfp4", fp4.FMT_MXINT4: "mxint4",
         fp4.FMT_NVINT4: "nvint4"}
SHAPES = [(69, 1056), (520, 4096)]
SHAPE_IDS = ["69x1056", "520x4096"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _prefilled(xd, fmt, rot, lay):
    """A Quantized output whose buffers start as 0xAA (unwritten bytes show)."""
    q = fp4.quantize(xd, fmt, rotate=rot, scale_layout=lay)
    q.codes.fill_(0xAA)
    q.scales.fill_(0xAA)
    q.global_scale.fill_(-1.0)
    return q


def _compare(q, rc, rs, rts, fmt, rot, what):
    torch.cuda.synchronize()
    gc, gs = codes_np(q), rowmajor_scales_np(q)
    if fmt not in fp4.MX_FORMATS:
        g = np.float32(q.global_scale.item())
        if rot:
            assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (what, g, rts)
        else:
            assert g == rts, (what, g, rts)
    if not rot:
        bad = np.argwhere(gc != rc)
        assert bad.size == 0, (what, bad[:4], gc[tuple(bad[:4].T)], rc[tuple(bad[:4].T)])
        bad = np.argwhere(gs != rs)
        assert bad.size == 0, (what, bad[:4], gs[tuple(bad[:4].T)], rs[tuple(bad[:4].T)])
    elif fmt in (fp4.FMT_MXINT4, fp4.FMT_NVINT4):
        assert_rotated_int4_close(gc, rc, gs, rs, what=what)
    else:
        assert_rotated_codes_close(gc, rc, gs, rs, what=what)


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
@pytest.mark.parametrize("rot", [False, True], ids=["plain", "rot"])
@pytest.mark.parametrize("fmt", [fp4.FMT_MXFP4, fp4.FMT_MXINT4], ids=["mxfp4", "mxint4"])
def test_edge_inputs_mx_every_bf16_kernel(fmt, rot, shape):
    rows, cols = shape
    # rotated: the butterfly of 32 values of 3e38 would leave fp32's range in
    # the partial sums, so the rotated tensor's big values are 3e36
    bits = workloads.edge_tensor(rows, cols, seed=21, family="mx", huge=3e36 if rot else 3e38)
    xh, xd = workloads.bf16_bits_to_f32(bits), to_dev_bf16(bits)
    say("edge mx", FNAME[fmt], "rot" if rot else "plain", shape)
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=rot)
    for lay in (fp4.SCALES_ROWMAJOR, fp4.SCALES_GEMM):
        q = _prefilled(xd, fmt, rot, lay)
        fp4.quantize(xd, fmt, rotate=rot, scale_layout=lay, out=q)
        _compare(q, rc, rs, rts, fmt, rot, "separate lay%d" % lay)
    outs = [_prefilled(xd, fmt, rot, lay) for lay in (fp4.SCALES_ROWMAJOR, fp4.SCALES_GEMM)]
    fp4.quantize_batch([dict(x=xd, fmt=fmt, rotate=rot, scale_layout=q.cfg.scale_layout, out=q)
                        for q in outs])
    for q in outs:
        _compare(q, rc, rs, rts, fmt, rot, "batch lay%d" % q.cfg.scale_layout)


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
@pytest.mark.parametrize("rot", [False, True], ids=["plain", "rot"])
@pytest.mark.parametrize("fmt", [fp4.FMT_NVFP4, fp4.FMT_NVINT4], ids=["nvfp4", "nvint4"])
def test_edge_inputs_nv_every_bf16_kernel(fmt, rot, shape):
    rows, cols = shape
    bits = workloads.edge_tensor(rows, cols, seed=22, family="nv", huge=1e4)
    xh, xd = workloads.bf16_bits_to_f32(bits), to_dev_bf16(bits)
    say("edge nv", FNAME[fmt], "rot" if rot else "plain", shape)
    rc, rs, rts = oracle.quantize(xh, fmt, rotate=rot)
    lay = fp4.SCALES_ROWMAJOR
    # the blocks scaled by 1e-5 and 1e-7 take subnormal and zero E4M3 scales
    assert np.any((rs > 0) & (rs < 8)) and np.any(rs == 0)
    q = _prefilled(xd, fmt, rot, lay)
    fp4.quantize(xd, fmt, rotate=rot, out=q)
    _compare(q, rc, rs, rts, fmt, rot, "two passes")
    assert fp4.fp4_quantize_one_pass_fits(q.cfg, fp4.DT_BF16, rows, cols, cols) == 1
    q = _prefilled(xd, fmt, rot, lay)
    fp4.quantize(xd, fmt, rotate=rot, out=q, one_pass=True, check_one_pass=True)
    _compare(q, rc, rs, rts, fmt, rot, "single pass")
    q = _prefilled(xd, fmt, rot, lay)
    fp4.quantize_batch([dict(x=xd, fmt=fmt, rotate=rot, out=q)])
    _compare(q, rc, rs, rts, fmt, rot, "batch")
    # the tensor scale given: the oracle's own, so the codes must match exactly
    rcg, rsg, _ = oracle.quantize(xh, fmt, rotate=rot, ts=rts)
    q = _prefilled(xd, fmt, rot, lay)
    fp4.quantize(xd, fmt, rotate=rot, out=q,
                 global_scale=torch.tensor([float(rts)], dtype=torch.float32, device="cuda"))
    _compare(q, rcg, rsg, rts, fmt, rot, "given scale")


def test_nvfp4_two_streams_match_separate_calls():
    """NVFP4 quantizations issued on two streams at once (two-pass, then
    single-pass on one stream beside two-pass on the other) give the results
    of the same calls made one after another: each stream has its own
    workspace, so no partial maxima or exchange slots are shared."""
    say("two streams")
    xs = [to_dev_bf16(workloads.cfg2_tensor(d, 5, rows=2048, cols=4096)) for d in ("gauss", "laplace")]
    ref = [fp4.quantize(x, fp4.FMT_NVFP4, rotate=r) for x in xs for r in (False, True)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for one_pass in (False, True):
        outs = []
        for rep in range(3):
            with torch.cuda.stream(s1):
                a = [fp4.quantize(xs[0], fp4.FMT_NVFP4, rotate=r, one_pass=one_pass) for r in (False, True)]
            with torch.cuda.stream(s2):
                b = [fp4.quantize(xs[1], fp4.FMT_NVFP4, rotate=r) for r in (False, True)]
            outs.append(a + b)
        torch.cuda.synchronize()
        for got in outs:
            for q, r in zip(got, ref):
                assert torch.equal(q.global_scale, r.global_scale)
                assert torch.equal(fp4.codes_view(q), fp4.codes_view(r))
                assert torch.equal(q.scales, r.scales)


def test_single_pass_give_up_check():
    """A clean single-pass call passes the give-up check and leaves the flag
    clear; with the flag set by the host (the kernel never clears it), the
    check raises FP4_ERR_EXCHANGE and re-zeroes the exchange region, after
    which calls pass again with unchanged results."""
    say("give-up check")
    x = to_dev_bf16(workloads.cfg2_tensor("gauss", 6, rows=512, cols=2048))
    q0 = fp4.quantize(x, fp4.FMT_NVFP4, one_pass=True, check_one_pass=True)
    cfg = fp4.qconfig(fp4.FMT_NVFP4)
    wsb = fp4.fp4_workspace_bytes(cfg, 512, 2048)
    ws = fp4._scratch_workspace(wsb, x.device, torch.cuda.current_stream().cuda_stream)
    off = fp4.EXCHANGE_FLAG_OFFSET
    assert int(ws[off:off + 4].view(torch.int32).item()) == 0
    ws[off:off + 4].view(torch.int32).fill_(1)
    with pytest.raises(fp4.FP4Error) as ei:
        fp4.quantize(x, fp4.FMT_NVFP4, one_pass=True, check_one_pass=True)
    assert ei.value.status == fp4.FP4_ERR_EXCHANGE
    assert int(ws[4096:].count_nonzero().item()) == 0
    q1 = fp4.quantize(x, fp4.FMT_NVFP4, one_pass=True, check_one_pass=True)
    torch.cuda.synchronize()
    assert torch.equal(q1.global_scale, q0.global_scale)
    assert torch.equal(fp4.codes_view(q1), fp4.codes_view(q0))

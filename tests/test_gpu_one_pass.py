"""Single-pass NVFP4 / NVINT4 quantize (FP4_GS_COMPUTE_ONE_PASS: the tensor
maximum and the encoding in one launch) against the two-pass path and the
oracle, bit for bit.

The single pass takes the maximum of the block values as the encoder forms
them (rotated in registers with the same butterflies), so codes, scale codes
and the tensor scale must equal the two-pass results exactly; non-rotated
results must also equal the oracle's, rotated ones stay within the
adjacent-mismatch budget.  Repeated calls and graph replays exercise the
exchange region's call numbering.
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

MASK = 0x0123456789ABCDEF0FEDCBA987654321

# (label, fmt, rotate, quantize keyword arguments)
CONFIGS = [
    ("nvfp4", fp4.FMT_NVFP4, False, {}),
    ("nvfp4-h16", fp4.FMT_NVFP4, True, {}),
    ("nvfp4-h16-signed", fp4.FMT_NVFP4, True, dict(signs=MASK)),
    ("nvfp4-mse", fp4.FMT_NVFP4, False, dict(rule=fp4.SCALE_MSE)),
    ("nvfp4-4over6-h16", fp4.FMT_NVFP4, True, dict(rule=fp4.SCALE_FOUR_OVER_SIX)),
    ("nvfp4-stochastic", fp4.FMT_NVFP4, False, dict(rounding=fp4.ROUND_STOCHASTIC, seed=(3, 4))),
    ("nvint4", fp4.FMT_NVINT4, False, {}),
    ("nvint4-h16", fp4.FMT_NVINT4, True, {}),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _bits(name):
    if name == "cfg2_gauss":
        return workloads.cfg2_tensor("gauss", 0)
    if name == "cfg2_laplace":
        return workloads.cfg2_tensor("laplace", 0)
    if name == "cfg3":
        return workloads.cfg3_tensor(0)  # 8192 x 4096: eight wave tiles per wave
    if name == "ragged":
        return workloads.cfg2_tensor("laplace", 9, rows=37, cols=4128)
    if name == "tiny_rows":
        return workloads.cfg2_tensor("gauss", 10, rows=3, cols=96)
    if name == "tiny_scale":
        g = workloads.bf16_bits_to_f32(workloads.cfg2_tensor("gauss", 13, rows=64, cols=1024))
        return workloads.to_bf16_bits((g * np.float32(2.0 ** -110)).astype(np.float32))
    raise KeyError(name)


def _same(qa, qb, what):
    ca, cb = codes_np(qa), codes_np(qb)
    bad = np.argwhere(ca != cb)
    assert bad.size == 0, (what, "codes", bad[:4])
    sa, sb = rowmajor_scales_np(qa), rowmajor_scales_np(qb)
    bad = np.argwhere(sa != sb)
    assert bad.size == 0, (what, "scales", bad[:4])
    ga, gb = qa.global_scale.item(), qb.global_scale.item()
    assert ga == gb or (np.isnan(ga) and np.isnan(gb)), (what, ga, gb)


def _prefilled(x, fmt, rot, kw):
    q = fp4.quantize(x, fmt, rotate=rot, **kw)
    q.codes.fill_(0xAA)
    q.scales.fill_(0xAA)
    q.global_scale.fill_(-1.0)
    return q


@pytest.mark.parametrize("case", ["cfg2_gauss", "cfg2_laplace", "cfg3", "ragged", "tiny_rows",
                                  "tiny_scale"])
def test_one_pass_equals_two_pass(case):
    b = _bits(case)
    x = to_dev_bf16(b)
    rows, cols = b.shape
    for label, fmt, rot, kw in CONFIGS:
        say("one pass vs two passes", case, label)
        cfg = fp4.qconfig(fmt, rot, **kw)
        assert fp4.fp4_quantize_one_pass_fits(cfg, fp4.DT_BF16, rows, cols, cols) == 1, (case, label)
        two = fp4.quantize(x, fmt, rotate=rot, **kw)
        one = fp4.quantize(x, fmt, rotate=rot, one_pass=True,
                           out=_prefilled(x, fmt, rot, kw), **kw)
        torch.cuda.synchronize()
        _same(one, two, (case, label))


@pytest.mark.parametrize("case", ["cfg2_laplace", "ragged", "tiny_scale"])
def test_one_pass_against_oracle(case):
    b = _bits(case)
    x = to_dev_bf16(b)
    xh = workloads.bf16_bits_to_f32(b)
    for label, fmt, rot, kw in CONFIGS:
        if kw:
            continue  # the searching rules, signs and stochastic rounding: covered above
        say("one pass vs oracle", case, label)
        rc, rs, rts = oracle.quantize(xh, fmt, rotate=rot)
        q = fp4.quantize(x, fmt, rotate=rot, one_pass=True, out=_prefilled(x, fmt, rot, {}))
        torch.cuda.synchronize()
        g = np.float32(q.global_scale.item())
        if not rot:
            assert np.array_equal(codes_np(q), rc) and np.array_equal(rowmajor_scales_np(q), rs)
            assert g == np.float32(rts)
            continue
        assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, (g, rts)
        if fmt == fp4.FMT_NVINT4:
            assert_rotated_int4_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)
        else:
            assert_rotated_codes_close(codes_np(q), rc, rowmajor_scales_np(q), rs, what=case)


def test_one_pass_repeated_calls_and_shapes():
    """Consecutive calls on one workspace, alternating shapes (different grid
    sizes, so slots of the larger grid go stale) and inputs: every call must
    match the two-pass result."""
    inputs = [to_dev_bf16(_bits(n)) for n in ("cfg2_gauss", "ragged", "cfg2_laplace", "tiny_rows")]
    for rep in range(3):
        for i, x in enumerate(inputs):
            say("one pass repeated", rep, i)
            two = fp4.quantize(x, fp4.FMT_NVFP4, rotate=bool(i & 1))
            one = fp4.quantize(x, fp4.FMT_NVFP4, rotate=bool(i & 1), one_pass=True)
            torch.cuda.synchronize()
            _same(one, two, (rep, i))


def test_one_pass_graph_replays():
    """The single pass captured in a HIP graph and replayed with eager work in
    between: each replay numbers its exchange anew and matches the two-pass
    result on whatever input the buffer holds."""
    say("one pass graph replays")
    src = [to_dev_bf16(_bits("cfg2_gauss")), to_dev_bf16(_bits("cfg2_laplace"))]
    x = src[0].clone()
    q = fp4.quantize(x, fp4.FMT_NVFP4, rotate=True, one_pass=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp4.quantize(x, fp4.FMT_NVFP4, rotate=True, one_pass=True, out=q)
    for r in range(4):
        x.copy_(src[r % 2])
        q.codes.fill_(0xAA)
        g.replay()
        ref = fp4.quantize(x, fp4.FMT_NVFP4, rotate=True)  # eager two-pass between replays
        torch.cuda.synchronize()
        _same(q, ref, ("replay", r))


def test_one_pass_workspace_init_through_the_c_abi():
    """A workspace full of garbage, prepared with fp4_workspace_init, then
    single-pass calls straight through the C ABI on it: each equals the
    two-pass result (the call numbering starts from the zeroed region)."""
    say("one pass workspace init")
    b = _bits("cfg2_laplace")
    x = to_dev_bf16(b)
    rows, cols = b.shape
    cfg = fp4.qconfig(fp4.FMT_NVFP4, True)
    wsb = fp4.fp4_workspace_bytes(cfg, rows, cols)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert fp4.fp4_workspace_init(ws.data_ptr(), wsb, stream) == 0
    ref = fp4.quantize(x, fp4.FMT_NVFP4, rotate=True)
    for rep in range(2):
        q = _prefilled(x, fp4.FMT_NVFP4, True, {})
        rc = fp4.fp4_quantize(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols, q.codes.data_ptr(),
                              q.scales.data_ptr(), q.global_scale.data_ptr(),
                              fp4.GS_COMPUTE_ONE_PASS, ws.data_ptr(), wsb, stream)
        assert rc == 0
        torch.cuda.synchronize()
        _same(q, ref, ("ws init", rep))
    assert int(ws[4096:4100].view(torch.int32).item()) == 2  # two calls numbered from zero


def test_one_pass_falls_back_when_it_does_not_fit():
    """Shapes and inputs the single launch does not take run the two passes:
    same results, and the fit query says so."""
    cfg = fp4.qconfig(fp4.FMT_NVFP4)
    rows, cols = 16384, 4096  # 64 M elements: past one launch's registers
    assert fp4.fp4_quantize_one_pass_fits(cfg, fp4.DT_BF16, rows, cols, cols) == 0
    assert fp4.fp4_quantize_one_pass_fits(cfg, fp4.DT_F32, 64, 1024, 1024) == 0
    assert fp4.fp4_quantize_one_pass_fits(fp4.qconfig(fp4.FMT_NVFP4, block_rows=16), fp4.DT_BF16,
                                          64, 1024, 1024) == 0
    assert fp4.fp4_quantize_one_pass_fits(fp4.qconfig(fp4.FMT_MXFP4), fp4.DT_BF16, 64, 1024, 1024) == 0
    b = workloads.cfg2_tensor("gauss", 21, rows=rows, cols=cols)
    x = to_dev_bf16(b)
    say("one pass fallback", rows, cols)
    _same(fp4.quantize(x, fp4.FMT_NVFP4, one_pass=True), fp4.quantize(x, fp4.FMT_NVFP4), "large")
    xf = x[:64].float()
    _same(fp4.quantize(xf, fp4.FMT_NVFP4, one_pass=True), fp4.quantize(xf, fp4.FMT_NVFP4), "fp32")
    torch.cuda.synchronize()

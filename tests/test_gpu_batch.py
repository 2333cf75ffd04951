"""fp4_quantize_batch (several quantizations, the mergeable ones in two
grouped launches) against separate fp4_quantize calls, bit for bit: codes,
scale bytes (whole buffers, padding included) and tensor scales.

The grouped kernel runs the same bodies with the same work split as the
separate launches; the tensor-maximum pass uses four waves per workgroup
instead of sixteen, which changes only how the maximum is partitioned, not
its value.  Non-rotated jobs are also checked against the oracle directly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import oracle
import workloads
from gpu_common import (assert_rotated_codes_close, codes_np, rowmajor_scales_np, say,
                        to_dev_bf16)

pytestmark = pytest.mark.gpu

MASK = 0x0123456789ABCDEF0FEDCBA987654321
MXG, MXR = fp4.SCALES_GEMM, fp4.SCALES_ROWMAJOR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _x(dist, seed, rows, cols, f32=False):
    x = to_dev_bf16(workloads.cfg2_tensor(dist, seed, rows=rows, cols=cols))
    return x.float() if f32 else x


# (label, fmt, quantize keyword arguments, gs_mode for NV formats)
MERGED = [
    ("mxfp4-gemm", fp4.FMT_MXFP4, dict(scale_layout=MXG), None),
    ("mxfp4-gemm-h32", fp4.FMT_MXFP4, dict(rotate=True, scale_layout=MXG), None),
    ("mxfp4-gemm-h32-signed", fp4.FMT_MXFP4, dict(rotate=True, scale_layout=MXG, signs=MASK), None),
    ("mxfp4-rowmajor", fp4.FMT_MXFP4, dict(scale_layout=MXR), None),
    ("mxfp4-rowmajor-h32", fp4.FMT_MXFP4, dict(rotate=True, scale_layout=MXR), None),
    ("mxint4-gemm-h32", fp4.FMT_MXINT4, dict(rotate=True, scale_layout=MXG), None),
    ("mxint4-rowmajor", fp4.FMT_MXINT4, dict(scale_layout=MXR), None),
    ("nvfp4", fp4.FMT_NVFP4, {}, fp4.GS_COMPUTE),
    ("nvfp4-h16", fp4.FMT_NVFP4, dict(rotate=True), fp4.GS_COMPUTE),
    ("nvfp4-h16-signed", fp4.FMT_NVFP4, dict(rotate=True, signs=MASK), fp4.GS_COMPUTE),
    ("nvfp4-one-pass", fp4.FMT_NVFP4, {}, fp4.GS_COMPUTE_ONE_PASS),
    ("nvfp4-given", fp4.FMT_NVFP4, dict(rotate=True), fp4.GS_GIVEN),
    ("nvint4", fp4.FMT_NVINT4, {}, fp4.GS_COMPUTE),
    ("nvint4-h16", fp4.FMT_NVINT4, dict(rotate=True), fp4.GS_COMPUTE),
]
# jobs the grouped launches do not take: they run as their own launches
SEPARATE = [
    ("nvfp4-mse", fp4.FMT_NVFP4, dict(rule=fp4.SCALE_MSE), fp4.GS_COMPUTE),
    ("nvfp4-4over6-h16", fp4.FMT_NVFP4, dict(rotate=True, rule=fp4.SCALE_FOUR_OVER_SIX), fp4.GS_COMPUTE),
    ("mxfp4-stochastic", fp4.FMT_MXFP4, dict(rounding=fp4.ROUND_STOCHASTIC, seed=(5, 6)), None),
    ("nvfp4-16x16", fp4.FMT_NVFP4, dict(block_rows=16), fp4.GS_COMPUTE),
    ("mxfp4-h128-signed", fp4.FMT_MXFP4, dict(rotate=128, scale_layout=MXG, signs=MASK), None),
    ("mxfp4-mse", fp4.FMT_MXFP4, dict(rule=fp4.SCALE_MSE, scale_layout=MXG), None),
]
GIVEN_TS = 3.0e-5


class Job:
    """One job: its input, the separate-call result and the batch outputs."""

    def __init__(self, label, fmt, kw, gs_mode, x):
        self.label, self.fmt, self.kw, self.gs_mode, self.x = label, fmt, dict(kw), gs_mode, x
        rows, cols = x.shape
        self.cfg = fp4.qconfig(fmt, kw.get("rotate", False), kw.get("scale_layout", MXR),
                               kw.get("rule", fp4.SCALE_ABSMAX), kw.get("rounding", fp4.ROUND_NEAREST),
                               kw.get("block_rows", 1), kw.get("signs", 0), kw.get("seed", (0, 0)))
        self.out = self._alloc()
        self.ref = self._alloc()
        if gs_mode == fp4.GS_GIVEN:
            self.out.global_scale.fill_(GIVEN_TS)

    def _alloc(self):
        rows, cols = self.x.shape
        codes = torch.full((max(fp4.fp4_codes_bytes(rows, cols), 16),), 0xAA, dtype=torch.uint8,
                           device="cuda")
        scales = torch.full((max(fp4.fp4_scales_bytes(self.cfg, rows, cols), 16),), 0xAA,
                            dtype=torch.uint8, device="cuda")
        gs = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        return fp4.Quantized(codes, scales, gs, self.cfg, rows, cols)

    def job(self):
        rows, cols = self.x.shape
        xdt = fp4.DT_F32 if self.x.dtype == torch.float32 else fp4.DT_BF16
        return fp4.quant_job(self.cfg, self.x.data_ptr(), xdt, rows, cols, self.x.stride(0),
                             self.out.codes.data_ptr(), self.out.scales.data_ptr(),
                             self.out.global_scale.data_ptr(),
                             fp4.GS_COMPUTE if self.gs_mode is None else self.gs_mode)

    def run_separately(self):
        kw = {k: v for k, v in self.kw.items()}
        gs = None
        if self.gs_mode == fp4.GS_GIVEN:
            gs = torch.full((1,), GIVEN_TS, dtype=torch.float32, device="cuda")
        fp4.quantize(self.x, self.fmt, global_scale=gs, out=self.ref, **kw)

    def check(self):
        a, b = self.out, self.ref
        assert torch.equal(a.codes, b.codes), (self.label, "codes")
        assert torch.equal(a.scales, b.scales), (self.label, "scale bytes")
        if self.fmt not in fp4.MX_FORMATS:
            ga, gb = a.global_scale.item(), b.global_scale.item()
            assert ga == gb, (self.label, ga, gb)


def _run_batch(jobs, stream=None):
    n = len(jobs)
    wsb = fp4.fp4_quantize_batch_workspace_bytes(n)
    ws = torch.full((max(wsb, 16),), 0xA5, dtype=torch.uint8, device="cuda")  # any contents
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = fp4.fp4_quantize_batch(n, fp4.job_array([j.job() for j in jobs]), ws.data_ptr(), wsb, st)
    assert rc == 0, fp4.status_str(rc)
    return ws


@pytest.mark.parametrize("shape", [(4096, 4096), (37, 4128), (3, 256)])
def test_batch_equals_separate_calls(shape):
    rows, cols = shape
    xg = _x("gauss", 31, rows, cols)
    xl = _x("laplace", 32, rows, cols)
    jobs = [Job(l, f, kw, m, xg if i % 2 == 0 else xl) for i, (l, f, kw, m) in enumerate(MERGED)]
    if rows < 4096:
        jobs += [Job(l, f, kw, m, xl) for (l, f, kw, m) in SEPARATE
                 if not (kw.get("block_rows") == 16 and rows % 16) and
                 not (kw.get("rotate") == 128 and cols % 128)]
        jobs.append(Job("nvfp4-fp32", fp4.FMT_NVFP4, dict(rotate=True), fp4.GS_COMPUTE,
                        _x("gauss", 33, rows, cols, f32=True)))
        # strided views (leading dimension cols + 64) in the grouped launches
        wide = _x("laplace", 34, rows, cols + 64)
        view = wide[:, :cols]
        jobs.append(Job("nvfp4-h16-strided", fp4.FMT_NVFP4, dict(rotate=True), fp4.GS_COMPUTE, view))
        jobs.append(Job("mxfp4-gemm-strided", fp4.FMT_MXFP4, dict(scale_layout=MXG), None, view))
    say("batch vs separate", shape, len(jobs), "jobs")
    ws = _run_batch(jobs)
    for j in jobs:
        j.run_separately()
    torch.cuda.synchronize()
    del ws
    for j in jobs:
        j.check()


def test_batch_many_jobs_and_empty_ones():
    """More than 16 grouped jobs per launch (several launches per phase),
    interleaved with empty jobs (NVFP4 with a computed scale writes ts = 0)."""
    jobs = []
    for i in range(21):
        label, fmt, kw, m = MERGED[i % len(MERGED)]
        jobs.append(Job("%s/%d" % (label, i), fmt, kw, m, _x("laplace", 40 + i, 5 + 7 * i, 512)))
        if i % 7 == 3:
            e = torch.empty(0, 512, dtype=torch.bfloat16, device="cuda")
            jobs.append(Job("empty/%d" % i, fp4.FMT_NVFP4, {}, fp4.GS_COMPUTE, e))
    say("batch of", len(jobs), "jobs")
    ws = _run_batch(jobs)
    for j in jobs:
        j.run_separately()
    torch.cuda.synchronize()
    del ws
    for j in jobs:
        j.check()
    assert jobs[4].label.startswith("empty") and jobs[4].out.global_scale.item() == 0.0


def test_batch_more_than_one_chunk():
    """70 grouped jobs: more than the 64 gathered per host-side chunk."""
    jobs = []
    for i in range(70):
        label, fmt, kw, m = MERGED[i % len(MERGED)]
        jobs.append(Job("%s/%d" % (label, i), fmt, kw, m, _x("gauss", 100 + i, 3 + (i % 5), 256)))
    say("batch of", len(jobs), "small jobs")
    ws = _run_batch(jobs)
    for j in jobs:
        j.run_separately()
    torch.cuda.synchronize()
    del ws
    for j in jobs:
        j.check()


def test_batch_against_oracle():
    """Non-rotated grouped jobs against the oracle directly (ragged shape)."""
    b = workloads.cfg2_tensor("laplace", 9, rows=37, cols=4128)
    x = to_dev_bf16(b)
    xh = workloads.bf16_bits_to_f32(b)
    picks = [(l, f, kw, m) for (l, f, kw, m) in MERGED
             if not kw.get("rotate") and m != fp4.GS_GIVEN]
    jobs = [Job(l, f, kw, m, x) for (l, f, kw, m) in picks]
    say("batch vs oracle", len(jobs), "jobs")
    ws = _run_batch(jobs)
    torch.cuda.synchronize()
    del ws
    for j in jobs:
        rc, rs, rts = oracle.quantize(xh, j.fmt, rotate=False)
        assert np.array_equal(codes_np(j.out), rc), j.label
        assert np.array_equal(rowmajor_scales_np(j.out), rs), j.label
        if j.fmt not in fp4.MX_FORMATS:
            assert np.float32(j.out.global_scale.item()) == np.float32(rts), j.label


def test_batch_full_size_step_against_oracle():
    """The benchmark's step as it is timed: one batch of the eight 4096 x 4096
    variants (two distributions x MXFP4 GEMM-layout / NVFP4 computing its
    scale x plain / block Hadamard), every job on its own input buffer, against
    the oracle on the whole tensors: bit-exact without rotation, within the
    adjacent-mismatch budget with it (tensor scale within one ulp)."""
    host = {d: workloads.cfg2_tensor(d, 0) for d in ("gauss", "laplace")}
    jobs = []
    for d in ("gauss", "laplace"):
        for fmt, kw, m in ((fp4.FMT_MXFP4, dict(scale_layout=MXG), None),
                           (fp4.FMT_NVFP4, {}, fp4.GS_COMPUTE)):
            for rot in (False, True):
                kw2 = dict(kw, rotate=rot)
                jobs.append((d, rot, Job("%s/%d/%s" % (d, fmt, rot), fmt, kw2, m,
                                         to_dev_bf16(host[d]))))
    say("full-size batch step", len(jobs), "jobs")
    ws = _run_batch([j for _, _, j in jobs])
    torch.cuda.synchronize()
    del ws
    for d, rot, j in jobs:
        rc, rs, rts = oracle.quantize(workloads.bf16_bits_to_f32(host[d]), j.fmt, rotate=rot)
        gc, gsc = codes_np(j.out), rowmajor_scales_np(j.out)
        if not rot:
            assert np.array_equal(gc, rc) and np.array_equal(gsc, rs), j.label
            if j.fmt == fp4.FMT_NVFP4:
                assert np.float32(j.out.global_scale.item()) == np.float32(rts), j.label
            continue
        assert_rotated_codes_close(gc, rc, gsc, rs, what=j.label)
        if j.fmt == fp4.FMT_NVFP4:
            g = np.float32(j.out.global_scale.item())
            assert abs(int(g.view(np.int32)) - int(np.float32(rts).view(np.int32))) <= 1, j.label


def test_batch_graph_replays():
    """The batch captured in a HIP graph, replayed on changing inputs with
    eager work in between: every replay equals separate calls on the input
    the buffers hold."""
    src = [_x("gauss", 50, 512, 4096), _x("laplace", 51, 512, 4096)]
    x = src[0].clone()
    jobs = [Job(l, f, kw, m, x) for (l, f, kw, m) in MERGED if m != fp4.GS_GIVEN]
    n = len(jobs)
    wsb = fp4.fp4_quantize_batch_workspace_bytes(n)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    arr = fp4.job_array([j.job() for j in jobs])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = fp4.fp4_quantize_batch(n, arr, ws.data_ptr(), wsb, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    for r in range(4):
        say("batch graph replay", r)
        x.copy_(src[r % 2])
        for j in jobs:
            j.out.codes.fill_(0xAA)
        g.replay()
        for j in jobs:
            j.run_separately()
        torch.cuda.synchronize()
        for j in jobs:
            j.check()


def test_quantize_batch_helper():
    """The Python helper gives what quantize() gives."""
    xg = _x("gauss", 60, 256, 1024)
    items = [dict(x=xg, fmt=fp4.FMT_MXFP4, rotate=True, scale_layout=MXG),
             dict(x=xg, fmt=fp4.FMT_NVFP4, rotate=True),
             dict(x=xg, fmt=fp4.FMT_NVFP4, global_scale=torch.tensor([2e-5], device="cuda"))]
    say("quantize_batch helper")
    outs = fp4.quantize_batch(items)
    for it, q in zip(items, outs):
        kw = {k: v for k, v in it.items() if k not in ("x", "fmt")}
        r = fp4.quantize(it["x"], it["fmt"], **kw)
        torch.cuda.synchronize()
        assert np.array_equal(codes_np(q), codes_np(r))
        assert np.array_equal(rowmajor_scales_np(q), rowmajor_scales_np(r))
        assert q.global_scale.item() == r.global_scale.item()

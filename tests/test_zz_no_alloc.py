"""fp4_quantize_noalloc: the quantize entry point whose NVFP4 scratch is a
static per-GPU device array instead of a caller workspace.  Called through
the C ABI and compared with fp4_quantize (the same configuration with a
workspace) bit for bit: codes, scales and tensor scale, for NVFP4 with the
tensor scale computed in two passes and in one, NVINT4, rotated and plain,
and MXFP4 (which needs no scratch), with row-major and tiled codes; two
calls in a row, the second with a smaller input, so that the static scratch
is reused."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import workloads

pytestmark = pytest.mark.gpu

CASES = [(fp4.FMT_NVFP4, False, fp4.GS_COMPUTE), (fp4.FMT_NVFP4, True, fp4.GS_COMPUTE),
         (fp4.FMT_NVFP4, False, fp4.GS_COMPUTE_ONE_PASS), (fp4.FMT_NVFP4, True, fp4.GS_COMPUTE_ONE_PASS),
         (fp4.FMT_NVINT4, True, fp4.GS_COMPUTE_ONE_PASS), (fp4.FMT_MXFP4, True, fp4.GS_COMPUTE)]
IDS = ["nvfp4-2pass", "nvfp4-h16-2pass", "nvfp4-1pass", "nvfp4-h16-1pass", "nvint4-h16-1pass",
       "mxfp4-h32"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _outputs(cfg, rows, cols, fill):
    """Output buffers: codes prefilled with `fill` (every byte is written);
    scales prefilled with 0xAA on both sides, since the GEMM layout's padding
    bytes are left as they are."""
    codes = torch.full((max(fp4.fp4_codes_bytes(rows, cols), 16),), fill, dtype=torch.uint8, device="cuda")
    scales = torch.full((max(fp4.fp4_scales_bytes(cfg, rows, cols), 16),), 0xAA, dtype=torch.uint8,
                        device="cuda")
    gs = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    return codes, scales, gs


@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("fmt,rot,mode", CASES, ids=IDS)
def test_noalloc_matches_workspace_entry_point(fmt, rot, mode, tiled):
    stream = torch.cuda.current_stream().cuda_stream
    lay = fp4.SCALES_GEMM if fmt in fp4.MX_FORMATS else fp4.SCALES_ROWMAJOR
    cfg = fp4.qconfig(fmt, rot, lay, code_layout=fp4.CODES_TILED if tiled else fp4.CODES_ROWMAJOR)
    # the second call smaller (tiled codes: multiples of 128 rows and columns)
    shapes = ((2048, 4096, 31), (256, 1024, 32)) if tiled else ((2048, 4096, 31), (37, 4128, 32))
    for rows, cols, seed in shapes:
        print("noalloc", fmt, rot, mode, tiled, rows, cols, flush=True)
        x = torch.from_numpy(workloads.cfg2_tensor("laplace", seed, rows=rows, cols=cols).view(np.int16))
        x = x.to("cuda").view(torch.bfloat16)
        ref = _outputs(cfg, rows, cols, 0xAA)
        got = _outputs(cfg, rows, cols, 0x55)
        wsb = fp4.fp4_workspace_bytes(cfg, rows, cols)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")
        rc = fp4.fp4_quantize(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols, ref[0].data_ptr(),
                              ref[1].data_ptr(), ref[2].data_ptr(), mode, ws.data_ptr(), wsb, stream)
        assert rc == fp4.FP4_OK
        rc = fp4.fp4_quantize_noalloc(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                      got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), mode,
                                      stream)
        assert rc == fp4.FP4_OK
        torch.cuda.synchronize()
        n = fp4.fp4_codes_bytes(rows, cols)
        ns = fp4.fp4_scales_bytes(cfg, rows, cols)
        assert torch.equal(got[0][:n], ref[0][:n])
        assert torch.equal(got[1][:ns], ref[1][:ns])
        if fmt not in fp4.MX_FORMATS:
            assert torch.equal(got[2], ref[2])


def test_noalloc_rejects_what_fp4_quantize_rejects():
    stream = torch.cuda.current_stream().cuda_stream
    cfg = fp4.qconfig(fp4.FMT_NVFP4)
    x = torch.zeros(4, 32, dtype=torch.bfloat16, device="cuda")
    c, s, g = _outputs(cfg, 4, 32, 0)
    assert fp4.fp4_quantize_noalloc(cfg, x.data_ptr(), fp4.DT_BF16, 4, 30, 32, c.data_ptr(),
                                    s.data_ptr(), g.data_ptr(), fp4.GS_COMPUTE, stream) \
        == fp4.FP4_ERR_INVALID_ARG
    assert fp4.fp4_quantize_noalloc(cfg, x.data_ptr(), fp4.DT_BF16, 4, 32, 32, c.data_ptr(),
                                    s.data_ptr(), None, fp4.GS_COMPUTE, stream) \
        == fp4.FP4_ERR_INVALID_ARG
    assert fp4.fp4_workspace_bytes(cfg, 4096, 4096) <= 8192  # the static scratch's size


@pytest.mark.parametrize("rot", [False, True], ids=["plain", "h16"])
def test_noalloc_one_pass_replayed_as_a_graph(rot):
    """The single-pass call (the exchange-repair kernel, then the quantize
    kernel) recorded in a HIP graph and replayed three times on changing
    inputs, with eager work between the replays: every replay equals the
    workspace entry point's result on the same input."""
    rows, cols = 1024, 2048
    cfg = fp4.qconfig(fp4.FMT_NVFP4, rot, fp4.SCALES_ROWMAJOR)
    xs = [torch.from_numpy(workloads.cfg2_tensor("laplace", 40 + i, rows=rows, cols=cols).view(np.int16))
          .to("cuda").view(torch.bfloat16) for i in range(3)]
    x = torch.empty_like(xs[0])
    got = _outputs(cfg, rows, cols, 0x55)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        h = torch.cuda.current_stream().cuda_stream
        assert fp4.fp4_quantize_noalloc(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                        got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                        fp4.GS_COMPUTE_ONE_PASS, h) == fp4.FP4_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        rc = fp4.fp4_quantize_noalloc(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                      got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                      fp4.GS_COMPUTE_ONE_PASS, h)
    assert rc == fp4.FP4_OK
    stream = torch.cuda.current_stream().cuda_stream
    wsb = fp4.fp4_workspace_bytes(cfg, rows, cols)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    n = fp4.fp4_codes_bytes(rows, cols)
    ns = fp4.fp4_scales_bytes(cfg, rows, cols)
    for i in range(3):
        print("noalloc graph replay", rot, i, flush=True)
        x.copy_(xs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _outputs(cfg, rows, cols, 0xAA)
        assert fp4.fp4_quantize(cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols, ref[0].data_ptr(),
                                ref[1].data_ptr(), ref[2].data_ptr(), fp4.GS_COMPUTE_ONE_PASS,
                                ws.data_ptr(), wsb, stream) == fp4.FP4_OK
        torch.cuda.synchronize()
        assert torch.equal(got[0][:n], ref[0][:n])
        assert torch.equal(got[1][:ns], ref[1][:ns])
        assert torch.equal(got[2], ref[2])
        assert bool(torch.isfinite(got[2]).all())

"""HIP-graph replay of the quantize and GEMM entry points (the benchmark times
graph replays).  The graph is recorded once and replayed several times with
eager work and synchronisations between replays; every replay must reproduce
the eager results byte for byte.  Nothing recorded clears memory with a
memset node: the calls launch kernels only.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4
import workloads
from gpu_common import say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _snapshot(qs, ys):
    return ([(q.codes.cpu().numpy().copy(), q.scales.cpu().numpy().copy(),
              q.global_scale.cpu().numpy().copy()) for q in qs],
            [y.float().cpu().numpy().copy() for y in ys])


def test_graph_replays_match_eager():
    say("case: graph replay, quantize MXFP4/NVFP4 (plain, rotated) 512x1024 + MXFP4/NVFP4 GEMMs")
    rows, cols, n = 512, 1024, 384
    xa = to_dev_bf16(workloads.cfg2_tensor("laplace", 3, rows=rows, cols=cols))
    xw = to_dev_bf16(workloads.cfg2_tensor("gauss", 4, rows=n, cols=cols))
    plans = [(fp4.FMT_MXFP4, False), (fp4.FMT_MXFP4, True), (fp4.FMT_NVFP4, False),
             (fp4.FMT_NVFP4, True)]
    qa = [fp4.quantize(xa, f, rotate=r, scale_layout=fp4.SCALES_GEMM) for f, r in plans]
    qw = [fp4.quantize(xw, f, rotate=r, scale_layout=fp4.SCALES_GEMM) for f, r in plans]
    ys = [torch.empty(rows, n, dtype=torch.bfloat16, device="cuda") for _ in plans]
    wss = []
    for (f, _), y in zip(plans, ys):
        wsb = fp4.fp4_gemm_workspace_bytes(f, rows, n, cols)
        wss.append(torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None)

    def step():
        for i, (f, r) in enumerate(plans):
            fp4.quantize(xa, f, rotate=r, scale_layout=fp4.SCALES_GEMM, out=qa[i])
            fp4.gemm(qa[i], qw[i], out=ys[i], workspace=wss[i])

    step()
    torch.cuda.synchronize()
    ref_q, ref_y = _snapshot(qa, ys)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # eager work between replays: wipe every output
        for q in qa:
            q.codes.fill_(0x5A)
            q.scales.fill_(0x5A)
            q.global_scale.fill_(-1.0)
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_q, got_y = _snapshot(qa, ys)
        for i, ((c0, s0, t0), (c1, s1, t1)) in enumerate(zip(ref_q, got_q)):
            assert np.array_equal(c0, c1), "replay %d plan %d codes differ" % (rep, i)
            assert np.array_equal(s0, s1), "replay %d plan %d scales differ" % (rep, i)
            if plans[i][0] == fp4.FMT_NVFP4:  # MXFP4 has no tensor scale to write
                assert np.array_equal(t0, t1), "replay %d plan %d tensor scale differs" % (rep, i)
        for i, (y0, y1) in enumerate(zip(ref_y, got_y)):
            assert np.array_equal(y0, y1), "replay %d plan %d GEMM output differs" % (rep, i)
    say("graph replays: 4 x identical to eager")

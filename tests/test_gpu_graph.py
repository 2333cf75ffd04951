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
        wss.append(torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None)

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


def test_graph_split_k_decode_replays():
    """Decode-shaped products split along K (partials in the workspace, then
    the fixed-order reduction): MXFP4, NVFP4 and weight-only GEMMs recorded in
    one graph, replayed with eager work between replays, every replay
    identical to the eager result; a second graph on the same workspaces as
    well."""
    say("case: graph replay, split-K decode GEMMs (M = 1 and 16, N = 4096, K = 8192)")
    K, n = 8192, 4096
    w = to_dev_bf16(workloads.gemm_weight(n, K, seed=6))
    a16 = to_dev_bf16(workloads.gemm_activation(16, K, seed=6))
    calls = []
    for f in (fp4.FMT_MXFP4, fp4.FMT_NVFP4):
        qw = fp4.quantize(w, f, scale_layout=fp4.SCALES_GEMM)
        for m in (1, 16):
            a = a16[:m]
            qa = fp4.quantize(a, f, scale_layout=fp4.SCALES_GEMM)
            assert fp4.fp4_gemm_workspace_bytes(f, m, n, K) > 0
            assert fp4.fp4_gemm_w4a16_workspace_bytes(f, m, n, K) > 0
            y = torch.empty(m, n, dtype=torch.float32, device="cuda")
            y4 = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
            ws = fp4.gemm_workspace(fp4.fp4_gemm_workspace_bytes(f, m, n, K), "cuda")
            ws4 = fp4.gemm_workspace(fp4.fp4_gemm_w4a16_workspace_bytes(f, m, n, K), "cuda")
            calls.append((lambda qa=qa, qw=qw, y=y, ws=ws: fp4.gemm(qa, qw, out=y, workspace=ws), y))
            calls.append((lambda a=a, qw=qw, y4=y4, ws4=ws4: fp4.gemm_w4a16(a, qw, out=y4, workspace=ws4), y4))

    def step():
        for fn, _ in calls:
            fn()

    step()
    torch.cuda.synchronize()
    ref = [y.float().cpu().numpy().copy() for _, y in calls]
    graphs = []
    for _ in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        graphs.append(g)
    for rep in range(6):
        for _, y in calls:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        torch.cuda.synchronize()
        for i, (_, y) in enumerate(calls):
            assert np.array_equal(y.float().cpu().numpy(), ref[i]), "replay %d call %d differs" % (rep, i)
        step()  # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
    say("split-K graph replays: 6 x identical to eager")

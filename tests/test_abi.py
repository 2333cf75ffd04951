"""C-ABI checks that need no GPU: the library loads, exports every function
that include/fp4.h declares, and rejects invalid arguments on the host before
any launch (fake device pointers are never dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

import fp4_microscaling_quantization_amd as fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced
MIS = 0x10004   # misaligned


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = fp4.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(fp4.EXPORTED)
    assert L.fp4_abi_version() == 5
    assert fp4.status_str(fp4.FP4_ERR_ALIGNMENT).startswith("misaligned")


@pytest.mark.parametrize("fmt", [fp4.FMT_MXFP4, fp4.FMT_NVFP4])
def test_sizes_give_the_formats_bits_per_element(fmt):
    cfg = fp4.qconfig(fmt)
    rows, cols = 64, 4096
    bits = 8 * (fp4.fp4_codes_bytes(rows, cols) + fp4.fp4_scales_bytes(cfg, rows, cols)) / (rows * cols)
    assert bits == {fp4.FMT_MXFP4: 4.25, fp4.FMT_NVFP4: 4.5}[fmt]
    assert fp4.fp4_workspace_bytes(cfg, rows, cols) == (8192 if fmt == fp4.FMT_NVFP4 else 0)


@pytest.mark.parametrize("rows,cols", [(1, 32), (31, 64), (33, 256), (100, 4096 + 128), (257, 288)])
def test_gemm_scale_layout_is_a_bijection(rows, cols):
    cfg = fp4.qconfig(fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM)
    size = fp4.fp4_scales_bytes(cfg, rows, cols)
    nb = cols // 32
    offs = [fp4.fp4_scale_offset(cfg, rows, cols, r, kb) for r in range(rows) for kb in range(nb)]
    assert min(offs) >= 0 and max(offs) < size
    assert len(set(offs)) == len(offs)
    # padded to 32 rows x 256 columns
    assert size == ((rows + 31) // 32) * ((cols + 255) // 256) * 256
    # the four scales one lane reads for consecutive 64-K MFMA steps share a dword
    if nb >= 8:
        d = [fp4.fp4_scale_offset(cfg, rows, cols, 0, kb) for kb in (0, 2, 4, 6)]
        assert d == [d[0], d[0] + 1, d[0] + 2, d[0] + 3] and d[0] % 4 == 0
    assert fp4.fp4_scale_offset(cfg, rows, cols, rows, 0) == -1
    assert fp4.fp4_scale_offset(cfg, rows, cols, 0, nb) == -1
    rm = fp4.qconfig(fp4.FMT_MXFP4)
    assert fp4.fp4_scale_offset(rm, rows, cols, rows - 1, nb - 1) == rows * nb - 1


def _q(cfg, **kw):
    a = dict(x=FAKE, xdt=fp4.DT_BF16, rows=64, cols=256, ldx=256, codes=FAKE, scales=FAKE,
             gs=FAKE, gs_mode=fp4.GS_COMPUTE, ws=FAKE, ws_bytes=8192, stream=None)
    a.update(kw)
    return fp4.fp4_quantize(cfg, a["x"], a["xdt"], a["rows"], a["cols"], a["ldx"], a["codes"],
                            a["scales"], a["gs"], a["gs_mode"], a["ws"], a["ws_bytes"], a["stream"])


def test_quantize_rejects_bad_arguments_on_host():
    mx = fp4.qconfig(fp4.FMT_MXFP4)
    nv = fp4.qconfig(fp4.FMT_NVFP4)
    E = fp4
    assert _q(mx, cols=48) == E.FP4_ERR_INVALID_ARG          # not a multiple of 32
    assert _q(nv, cols=40) == E.FP4_ERR_INVALID_ARG          # not a multiple of 16
    assert _q(mx, ldx=128) == E.FP4_ERR_INVALID_ARG          # ldx < cols
    assert _q(mx, rows=-1) == E.FP4_ERR_INVALID_ARG
    assert _q(mx, xdt=7) == E.FP4_ERR_INVALID_ARG
    assert _q(mx, x=MIS) == E.FP4_ERR_ALIGNMENT
    assert _q(mx, codes=MIS) == E.FP4_ERR_ALIGNMENT
    assert _q(mx, ldx=260) == E.FP4_ERR_ALIGNMENT            # 520-byte rows
    assert _q(mx, x=None) == E.FP4_ERR_INVALID_ARG
    assert _q(mx, scales=None) == E.FP4_ERR_INVALID_ARG
    assert _q(nv, gs=None) == E.FP4_ERR_INVALID_ARG
    assert _q(nv, ws=None) == E.FP4_ERR_WORKSPACE
    assert _q(nv, ws_bytes=8) == E.FP4_ERR_WORKSPACE
    assert _q(nv, gs_mode=5) == E.FP4_ERR_INVALID_ARG
    assert _q(nv, ws_bytes=2048) == E.FP4_ERR_WORKSPACE
    # the single-pass exchange region holds 64-bit slots
    assert _q(nv, gs_mode=fp4.GS_COMPUTE_ONE_PASS, ws=FAKE + 4) == E.FP4_ERR_ALIGNMENT
    assert _q(nv, gs_mode=fp4.GS_COMPUTE_ONE_PASS, ws=None) == E.FP4_ERR_WORKSPACE
    assert _q(nv, gs_mode=fp4.GS_COMPUTE_ONE_PASS, gs=None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_workspace_init(None, 8192, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_workspace_init(FAKE, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_workspace_init(FAKE + 4, 8192, None) == E.FP4_ERR_ALIGNMENT
    assert fp4.fp4_workspace_init(FAKE, 8190, None) == E.FP4_ERR_ALIGNMENT
    assert fp4.fp4_global_scale(mx, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, 2048, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_global_scale(nv, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, None, 0, None) == E.FP4_ERR_WORKSPACE
    assert fp4.fp4_global_scale(nv, MIS, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, 2048, None) == E.FP4_ERR_ALIGNMENT
    assert fp4.fp4_global_scale(nv, FAKE, fp4.DT_BF16, 64, 256, 256, None, FAKE, 256, None) == E.FP4_ERR_INVALID_ARG
    bad = fp4.QConfig(fp4.FMT_MXFP4, 16, 0, 0, 0)
    assert _q(bad) == E.FP4_ERR_INVALID_ARG                  # MXFP4 block must be 32
    bad = fp4.QConfig(fp4.FMT_MXFP4, 32, 16, 0, 0)
    assert _q(bad) == E.FP4_ERR_INVALID_ARG                  # rotation size must equal block
    ok = fp4.QConfig(fp4.FMT_NVFP4, 16, 0, fp4.SCALE_MSE, 0)
    assert fp4.fp4_scales_bytes(ok, 64, 256) == 64 * 16       # the MSE rule is a valid config
    ok = fp4.QConfig(fp4.FMT_NVFP4, 16, 0, fp4.SCALE_FOUR_OVER_SIX, 0)
    assert fp4.fp4_scales_bytes(ok, 64, 256) == 64 * 16
    bad = fp4.QConfig(fp4.FMT_MXFP4, 32, 0, fp4.SCALE_FOUR_OVER_SIX, 0)
    assert _q(bad) == E.FP4_ERR_UNSUPPORTED                  # Four Over Six is NVFP4's
    bad = fp4.QConfig(fp4.FMT_NVFP4, 16, 0, 3, 0)
    assert _q(bad) == E.FP4_ERR_INVALID_ARG                  # no such rule
    # rotation sizes, stochastic rounding and 16x16 blocks
    assert _q(fp4.qconfig(fp4.FMT_MXFP4, 128), cols=384) == E.FP4_ERR_INVALID_ARG  # cols % 128
    assert _q(fp4.qconfig(fp4.FMT_NVFP4, 64)) == E.FP4_ERR_INVALID_ARG    # NV rotations are 16-point
    assert _q(fp4.qconfig(fp4.FMT_MXFP4, 48)) == E.FP4_ERR_INVALID_ARG
    assert _q(fp4.qconfig(fp4.FMT_NVFP4, rounding=2)) == E.FP4_ERR_INVALID_ARG
    assert _q(fp4.qconfig(fp4.FMT_NVFP4, rounding=1, rule=fp4.SCALE_MSE)) == E.FP4_ERR_UNSUPPORTED
    assert _q(fp4.qconfig(fp4.FMT_NVINT4, rounding=1)) == E.FP4_ERR_UNSUPPORTED
    assert _q(fp4.qconfig(fp4.FMT_NVFP4, block_rows=8)) == E.FP4_ERR_INVALID_ARG
    assert _q(fp4.qconfig(fp4.FMT_MXFP4, block_rows=16)) == E.FP4_ERR_UNSUPPORTED
    assert _q(fp4.qconfig(fp4.FMT_NVFP4, True, block_rows=16)) == E.FP4_ERR_UNSUPPORTED
    assert fp4.fp4_scales_bytes(fp4.qconfig(fp4.FMT_NVFP4, block_rows=16), 64, 256) == 64 * 16
    assert fp4.fp4_scales_bytes(fp4.qconfig(fp4.FMT_MXFP4, 128, fp4.SCALES_GEMM, signs=5), 64, 256) == 512
    assert ctypes.sizeof(fp4.QConfig) == 56
    # INT4-element formats: the MX / NV layouts, absmax scales only
    mxi = fp4.qconfig(fp4.FMT_MXINT4, scale_layout=fp4.SCALES_GEMM)
    nvi = fp4.qconfig(fp4.FMT_NVINT4)
    assert fp4.fp4_scales_bytes(mxi, 64, 256) == 2 * 256
    assert fp4.fp4_workspace_bytes(nvi, 64, 256) == 8192 and fp4.fp4_workspace_bytes(mxi, 64, 256) == 0
    assert _q(fp4.QConfig(fp4.FMT_MXINT4, 16, 0, 0, 0)) == E.FP4_ERR_INVALID_ARG
    assert _q(fp4.QConfig(fp4.FMT_NVINT4, 16, 0, fp4.SCALE_MSE, 0)) == E.FP4_ERR_UNSUPPORTED
    assert _q(nvi, gs=None) == E.FP4_ERR_INVALID_ARG
    assert _q(fp4.QConfig(4, 16, 0, 0, 0)) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_global_scale(mxi, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, 2048, None) == E.FP4_ERR_INVALID_ARG
    bad = fp4.QConfig(3, 32, 0, 0, 0)
    assert _q(bad) == E.FP4_ERR_INVALID_ARG
    bad = fp4.QConfig(fp4.FMT_MXFP4, 32, 0, 0, 9)
    assert _q(bad) == E.FP4_ERR_INVALID_ARG
    # an empty MXFP4 tensor is a no-op that launches nothing
    assert _q(mx, rows=0, x=None, codes=None, scales=None) == E.FP4_OK
    assert _q(mx, cols=0, x=None, codes=None, scales=None) == E.FP4_OK


def _job(cfg, rows=64, cols=256, ldx=256, x=FAKE, xdt=None, codes=FAKE, scales=FAKE, gs=FAKE,
         gs_mode=fp4.GS_COMPUTE):
    return fp4.quant_job(cfg, x, fp4.DT_BF16 if xdt is None else xdt, rows, cols, ldx, codes,
                         scales, gs, gs_mode)


def test_quantize_batch_rejects_bad_arguments_on_host():
    """Every job is checked before anything is launched; the first failing
    job's status comes back (fake pointers: a launch would fault, so reaching
    one would crash this CPU test)."""
    E = fp4
    mx = fp4.qconfig(fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM)
    nv = fp4.qconfig(fp4.FMT_NVFP4, True)
    assert ctypes.sizeof(fp4.QuantJob) == 128
    assert fp4.fp4_quantize_batch_workspace_bytes(0) == 0
    assert fp4.fp4_quantize_batch_workspace_bytes(3) == 3 * 2048
    assert fp4.fp4_quantize_batch_workspace_bytes(-1) == 0
    good = [_job(mx), _job(nv)]

    def run(jobs, ws=FAKE, ws_bytes=None, n=None):
        n = len(jobs) if n is None else n
        wsb = 2048 * len(jobs) if ws_bytes is None else ws_bytes
        return fp4.fp4_quantize_batch(n, fp4.job_array(jobs) if jobs else None, ws, wsb, None)

    assert run([]) == E.FP4_OK                                   # n == 0: nothing to do
    assert fp4.fp4_quantize_batch(-1, None, None, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_quantize_batch(2, None, FAKE, 4096, None) == E.FP4_ERR_INVALID_ARG
    # a bad job anywhere stops the whole batch, with that job's status
    assert run(good + [_job(mx, cols=48)]) == E.FP4_ERR_INVALID_ARG
    assert run(good + [_job(mx, x=MIS)]) == E.FP4_ERR_ALIGNMENT
    assert run(good + [_job(mx, codes=MIS)]) == E.FP4_ERR_ALIGNMENT
    assert run(good + [_job(nv, gs=None)]) == E.FP4_ERR_INVALID_ARG
    assert run(good + [_job(nv, gs_mode=7)]) == E.FP4_ERR_INVALID_ARG
    assert run(good + [_job(mx, xdt=9)]) == E.FP4_ERR_INVALID_ARG
    assert run(good + [_job(fp4.qconfig(fp4.FMT_MXFP4, block_rows=16))]) == E.FP4_ERR_UNSUPPORTED
    # workspace: 2048 bytes per job, 4-byte aligned, when a job computes a tensor scale
    assert run(good, ws=None) == E.FP4_ERR_WORKSPACE
    assert run(good, ws_bytes=2 * 2048 - 4) == E.FP4_ERR_WORKSPACE
    assert run(good, ws=FAKE + 2) == E.FP4_ERR_ALIGNMENT
    # all jobs empty: valid, and no workspace is needed for the MX formats
    assert run([_job(mx, rows=0, x=None, codes=None, scales=None)], ws=None) == E.FP4_OK


def test_dequantize_error_sums_and_relayout_reject_bad_arguments():
    mx = fp4.qconfig(fp4.FMT_MXFP4)
    nv = fp4.qconfig(fp4.FMT_NVFP4)
    E = fp4
    assert fp4.fp4_dequantize(mx, FAKE, FAKE, None, 4, 40, FAKE, fp4.DT_F32, 40, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_dequantize(mx, MIS, FAKE, None, 4, 64, FAKE, fp4.DT_F32, 64, 0, None) == E.FP4_ERR_ALIGNMENT
    assert fp4.fp4_dequantize(mx, FAKE, FAKE, None, 4, 64, FAKE, fp4.DT_F32, 32, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_dequantize(nv, FAKE, FAKE, None, 4, 64, FAKE, fp4.DT_F32, 64, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_dequantize(mx, FAKE, FAKE, None, 0, 64, None, fp4.DT_F32, 64, 0, None) == E.FP4_OK
    wsb = fp4.fp4_error_workspace_bytes(mx, 64, 256)
    assert wsb > 0
    assert fp4.fp4_error_sums(mx, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, None, FAKE, FAKE, wsb - 8, None) == E.FP4_ERR_WORKSPACE
    assert fp4.fp4_error_sums(mx, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, None, None, FAKE, wsb, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_error_sums(mx, FAKE, fp4.DT_BF16, 64, 256, 256, FAKE, FAKE, None, FAKE + 4, FAKE, wsb, None) == E.FP4_ERR_ALIGNMENT
    assert fp4.fp4_scales_to_gemm_layout(nv, FAKE, 4, 64, FAKE, None) == E.FP4_ERR_UNSUPPORTED
    assert fp4.fp4_scales_to_gemm_layout(mx, FAKE, 4, 40, FAKE, None) == E.FP4_ERR_INVALID_ARG


def _g(**kw):
    a = dict(fmt=fp4.FMT_MXFP4, M=64, N=64, K=256, a=FAKE, asc=FAKE, ags=FAKE, b=FAKE, bsc=FAKE,
             bgs=FAKE, y=FAKE, ydt=fp4.DT_BF16, ldy=64, ws=None, wsb=0, stream=None)
    a.update(kw)
    return fp4.fp4_gemm(a["fmt"], a["M"], a["N"], a["K"], a["a"], a["asc"], a["ags"], a["b"],
                        a["bsc"], a["bgs"], a["y"], a["ydt"], a["ldy"], a["ws"], a["wsb"], a["stream"])


def test_gemm_rejects_bad_arguments_on_host():
    E = fp4
    assert _g(K=96) == E.FP4_ERR_UNSUPPORTED                 # K must be a multiple of 128
    assert _g(M=-1) == E.FP4_ERR_INVALID_ARG
    assert _g(fmt=7) == E.FP4_ERR_INVALID_ARG
    assert _g(ldy=32) == E.FP4_ERR_INVALID_ARG
    assert _g(ydt=9) == E.FP4_ERR_INVALID_ARG
    assert _g(a=MIS) == E.FP4_ERR_ALIGNMENT
    assert _g(bsc=FAKE + 2) == E.FP4_ERR_ALIGNMENT
    assert _g(asc=FAKE + 4) == E.FP4_ERR_ALIGNMENT  # scales: 16-byte aligned
    assert _g(y=None) == E.FP4_ERR_INVALID_ARG
    assert _g(b=None) == E.FP4_ERR_INVALID_ARG
    assert _g(fmt=fp4.FMT_NVFP4, ags=None) == E.FP4_ERR_INVALID_ARG
    assert _g(M=0, y=None) == E.FP4_OK                       # empty output: nothing to do
    assert _g(fmt=fp4.FMT_MXINT4, K=384) == E.FP4_ERR_UNSUPPORTED  # INT4 elements: K % 256
    assert _g(fmt=fp4.FMT_NVINT4, bgs=None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_gemm_workspace_bytes(fp4.FMT_NVINT4, 1, 8192, 28672) > 0
    assert fp4.fp4_gemm_workspace_bytes(fp4.FMT_MXFP4, 1, 8192, 28672) > 0
    assert fp4.fp4_gemm_workspace_bytes(fp4.FMT_MXFP4, 4096, 4096, 4096) == 0
    assert _g(ws=FAKE + 8, wsb=1 << 20) == E.FP4_ERR_ALIGNMENT  # split-K partials: 16-byte aligned


def test_tiled_code_layout_is_checked_on_host():
    """FP4_CODES_TILED needs rows and cols that are multiples of 128, tiled B
    operands N % 128 == 0; unknown layout values and fmt bits are rejected."""
    E = fp4
    for fmt in (fp4.FMT_MXFP4, fp4.FMT_NVFP4, fp4.FMT_MXINT4, fp4.FMT_NVINT4):
        t = fp4.qconfig(fmt, code_layout=fp4.CODES_TILED)
        assert fp4.fp4_scales_bytes(t, 128, 256) == fp4.fp4_scales_bytes(fp4.qconfig(fmt), 128, 256)
        assert fp4.fp4_scales_bytes(t, 64, 256) == 0
        assert fp4.fp4_scales_bytes(t, 128, 192) == 0
        assert _q(t, rows=64) == E.FP4_ERR_INVALID_ARG
        assert _q(t, rows=128, cols=192, ldx=192) == E.FP4_ERR_INVALID_ARG
        assert fp4.fp4_dequantize(t, FAKE, FAKE, FAKE, 64, 256, FAKE, fp4.DT_F32, 256, 0, None) == E.FP4_ERR_INVALID_ARG
    assert fp4.fp4_scales_bytes(fp4.qconfig(fp4.FMT_MXFP4, code_layout=2), 128, 256) == 0
    bt = fp4.GEMM_B_TILED
    assert _g(fmt=fp4.FMT_MXFP4 | bt, N=64) == E.FP4_ERR_INVALID_ARG      # N % 128
    assert _g(fmt=fp4.FMT_NVFP4 | bt, N=192, ldy=192) == E.FP4_ERR_INVALID_ARG
    assert _g(fmt=fp4.FMT_MXFP4 | 0x200) == E.FP4_ERR_INVALID_ARG         # unknown flag bits
    assert _g(fmt=fp4.FMT_MXFP4 | bt, N=128, ldy=128, M=0, y=None) == E.FP4_OK
    assert _w(fmt=fp4.FMT_MXFP4 | bt, N=64) == E.FP4_ERR_INVALID_ARG
    for fmt in (fp4.FMT_MXFP4, fp4.FMT_NVFP4, fp4.FMT_MXINT4, fp4.FMT_NVINT4):
        for M, N, K in ((1, 28672, 8192), (16, 8192, 28672), (4096, 4096, 4096)):
            assert fp4.fp4_gemm_workspace_bytes(fmt | bt, M, N, K) == fp4.fp4_gemm_workspace_bytes(fmt, M, N, K)
            assert (fp4.fp4_gemm_w4a16_workspace_bytes(fmt | bt, M, N, K)
                    == fp4.fp4_gemm_w4a16_workspace_bytes(fmt, M, N, K))


def _w(**kw):
    a = dict(fmt=fp4.FMT_MXFP4, M=16, N=64, K=512, a=FAKE, lda=512, b=FAKE, bsc=FAKE, bgs=FAKE,
             y=FAKE, ydt=fp4.DT_BF16, ldy=64, ws=None, wsb=0, stream=None)
    a.update(kw)
    return fp4.fp4_gemm_w4a16(a["fmt"], a["M"], a["N"], a["K"], a["a"], a["lda"], a["b"], a["bsc"],
                              a["bgs"], a["y"], a["ydt"], a["ldy"], a["ws"], a["wsb"], a["stream"])


def test_gemm_w4a16_rejects_bad_arguments_on_host():
    E = fp4
    assert _w(K=128) == E.FP4_ERR_UNSUPPORTED                # K must be a multiple of 256
    assert _w(fmt=7) == E.FP4_ERR_INVALID_ARG
    assert _w(M=-1) == E.FP4_ERR_INVALID_ARG
    assert _w(ldy=32) == E.FP4_ERR_INVALID_ARG
    assert _w(lda=256) == E.FP4_ERR_INVALID_ARG              # lda < K
    assert _w(ydt=9) == E.FP4_ERR_INVALID_ARG
    assert _w(a=MIS) == E.FP4_ERR_ALIGNMENT
    assert _w(lda=516) == E.FP4_ERR_ALIGNMENT                # 1032-byte activation rows
    assert _w(b=MIS) == E.FP4_ERR_ALIGNMENT
    assert _w(bsc=FAKE + 4) == E.FP4_ERR_ALIGNMENT
    assert _w(ws=FAKE + 4, wsb=1 << 20) == E.FP4_ERR_ALIGNMENT
    assert _w(a=None) == E.FP4_ERR_INVALID_ARG
    assert _w(y=None) == E.FP4_ERR_INVALID_ARG
    assert _w(fmt=fp4.FMT_NVFP4, bgs=None) == E.FP4_ERR_INVALID_ARG
    assert _w(M=0, y=None) == E.FP4_OK                       # empty output: nothing to do
    assert _w(N=0, y=None) == E.FP4_OK
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_MXFP4, 1, 8192, 28672) > 0
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_NVFP4, 16, 4096, 8192) > 0
    # 224 column tiles of 128 already fill the GPU: no split
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_NVFP4, 16, 28672, 8192) == 0
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_MXFP4, 1, 8192, 1000) == 0
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_MXFP4, 4096, 4096, 4096) == 0
    assert fp4.fp4_gemm_w4a16_workspace_bytes(fp4.FMT_MXINT4, 1, 8192, 28672) > 0
    assert _w(fmt=fp4.FMT_NVINT4, bgs=None) == E.FP4_ERR_INVALID_ARG

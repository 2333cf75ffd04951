"""Python-binding checks that need no GPU: the argument checks of gemm() and
gemm_w4a16(), the workspace size offered to the C ABI, the per-stream
workspace caches and the single-pass give-up detection.  The C-ABI product
calls are replaced by recorders, so nothing is launched."""
import pytest

torch = pytest.importorskip("torch")

import fp4_microscaling_quantization_amd as fp4


def _operand(fmt, rows, K, layout=fp4.SCALES_GEMM, rotate=False, signs=0):
    cfg = fp4.qconfig(fmt, rotate, layout, signs=signs)
    codes = torch.zeros(max(rows * K // 2, 16), dtype=torch.uint8)
    scales = torch.zeros(max(fp4.fp4_scales_bytes(cfg, rows, K), 16), dtype=torch.uint8)
    return fp4.Quantized(codes, scales, torch.zeros(1), cfg, rows, K)


@pytest.fixture
def recorder(monkeypatch):
    calls = []

    def rec(name):
        def f(*args):
            calls.append((name, args))
            return fp4.FP4_OK
        return f

    monkeypatch.setattr(fp4, "fp4_gemm", rec("fp4_gemm"))
    monkeypatch.setattr(fp4, "fp4_gemm_w4a16", rec("fp4_gemm_w4a16"))
    monkeypatch.setattr(fp4, "_stream", lambda: 0)
    return calls


@pytest.mark.parametrize("nbytes", [0, 64, 5000])
def test_gemm_offers_the_workspace_buffers_own_size(recorder, nbytes):
    """The size passed as ws_bytes is the buffer's, not the size the call
    needs: a buffer that is too small then runs unsplit instead of being
    written past its end."""
    a, b = _operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_MXFP4, 4096, 1024)
    ws = torch.zeros(nbytes, dtype=torch.uint8)
    fp4.gemm(a, b, out_dtype=torch.float32, workspace=ws)
    name, args = recorder[-1]
    assert name == "fp4_gemm" and args[-2] == nbytes
    w = torch.empty(64, 1024, dtype=torch.bfloat16)
    fp4.gemm_w4a16(w, b, out_dtype=torch.float32, workspace=ws)
    name, args = recorder[-1]
    assert name == "fp4_gemm_w4a16" and args[-2] == nbytes


def test_gemm_without_workspace_offers_none_or_the_cached_one(recorder):
    a, b = _operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_MXFP4, 4096, 1024)
    need = fp4.fp4_gemm_workspace_bytes(fp4.FMT_MXFP4, 64, 4096, 1024)
    fp4.gemm(a, b, out_dtype=torch.float32)
    args = recorder[-1][1]
    if need:
        assert args[-2] >= need and args[-3] is not None
    else:
        assert args[-2] == 0 and args[-3] is None


def test_gemm_rejects_a_workspace_of_another_type(recorder):
    a, b = _operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_MXFP4, 128, 1024)
    with pytest.raises(ValueError):
        fp4.gemm(a, b, workspace=torch.zeros(16, dtype=torch.float32))
    assert not recorder


def test_gemm_rejects_row_major_mx_scales(recorder):
    a = _operand(fp4.FMT_MXFP4, 64, 1024, layout=fp4.SCALES_ROWMAJOR)
    b = _operand(fp4.FMT_MXFP4, 128, 1024)
    with pytest.raises(ValueError, match="GEMM"):
        fp4.gemm(a, b)
    with pytest.raises(ValueError, match="GEMM"):
        fp4.gemm(b, a)
    with pytest.raises(ValueError, match="GEMM"):
        fp4.gemm_w4a16(torch.empty(8, 1024, dtype=torch.bfloat16), a)
    # NVFP4: the two layouts coincide, both are accepted
    fp4.gemm(_operand(fp4.FMT_NVFP4, 64, 1024, layout=fp4.SCALES_ROWMAJOR),
             _operand(fp4.FMT_NVFP4, 128, 1024))
    assert len(recorder) == 1


@pytest.mark.parametrize("rb,sb", [((True, 0), (False, 0)), ((True, 5), (True, 0)),
                                   ((64, 0), (32, 0)), ((128, 3), (128, 7))])
def test_gemm_rejects_differently_rotated_operands(recorder, rb, sb):
    a = _operand(fp4.FMT_MXFP4, 64, 1024, rotate=rb[0], signs=rb[1])
    b = _operand(fp4.FMT_MXFP4, 128, 1024, rotate=sb[0], signs=sb[1])
    with pytest.raises(ValueError, match="rotation"):
        fp4.gemm(a, b)
    fp4.gemm(a, _operand(fp4.FMT_MXFP4, 128, 1024, rotate=rb[0], signs=rb[1]))
    assert len(recorder) == 1


def test_gemm_rejects_mismatched_formats_and_k(recorder):
    with pytest.raises(ValueError):
        fp4.gemm(_operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_NVFP4, 64, 1024))
    with pytest.raises(ValueError):
        fp4.gemm(_operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_MXFP4, 64, 2048))
    assert not recorder


@pytest.mark.parametrize("bad", ["shape", "dtype", "stride", "overlap"])
def test_gemm_rejects_an_unusable_output(recorder, bad):
    a, b = _operand(fp4.FMT_MXFP4, 64, 1024), _operand(fp4.FMT_MXFP4, 128, 1024)
    out = {"shape": torch.empty(64, 127),
           "dtype": torch.empty(64, 128, dtype=torch.float16),
           "stride": torch.empty(128, 64).t(),
           "overlap": torch.empty(64 * 128 + 64).as_strided((64, 128), (64, 1))}[bad]
    with pytest.raises(ValueError):
        fp4.gemm(a, b, out=out)
    with pytest.raises(ValueError):
        fp4.gemm_w4a16(torch.empty(64, 1024, dtype=torch.bfloat16), b, out=out)
    assert not recorder
    # a row-strided view of a wider buffer is a valid output (ldy > N)
    fp4.gemm(a, b, out=torch.empty(64, 200)[:, :128])
    assert recorder[-1][1][12] == 200


def test_scratch_workspaces_are_per_stream():
    w1 = fp4._scratch_workspace(8192, torch.device("cpu"), 11)
    w2 = fp4._scratch_workspace(8192, torch.device("cpu"), 12)
    assert w1.data_ptr() != w2.data_ptr()
    assert fp4._scratch_workspace(8192, torch.device("cpu"), 11) is w1
    assert int(w1.count_nonzero()) == 0  # the exchange region starts at zero
    g1 = fp4._gemm_workspace(1000, torch.device("cpu"), 11)
    g2 = fp4._gemm_workspace(1000, torch.device("cpu"), 12)
    assert g1.data_ptr() != g2.data_ptr()
    assert fp4._gemm_workspace(500, torch.device("cpu"), 11) is g1
    assert fp4._gemm_workspace(4000, torch.device("cpu"), 11).numel() >= 4000


def test_one_pass_give_up_detection():
    assert not fp4.one_pass_gave_up(0, 0.25)
    assert not fp4.one_pass_gave_up(0, 0.0)
    assert fp4.one_pass_gave_up(1, 0.25)          # the flag, with a finite scale
    assert fp4.one_pass_gave_up(0, float("nan"))  # the NaN scale alone
    assert fp4.EXCHANGE_FLAG_OFFSET == 4100
    assert fp4.status_str(fp4.FP4_ERR_EXCHANGE).startswith("single-pass")

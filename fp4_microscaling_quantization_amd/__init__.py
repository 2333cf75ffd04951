"""MI355X (gfx950) microscaling FP4: Python binding over ``libfp4.so``.

The binding only marshals arguments into the C ABI declared in
``include/fp4.h``; every step of quantization, dequantization, error sums and
the block-scaled GEMM runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream.  There is no fallback: if the library
is not built, or no GPU is present, the calls raise.

Low-level names mirror the C ABI (``fp4_quantize``, ``fp4_dequantize``,
``fp4_error_sums``, ``fp4_gemm``, ``fp4_scales_to_gemm_layout`` and the size /
offset helpers); ``quantize``, ``dequantize``, ``error_sums`` and ``gemm``
allocate their outputs with torch and call them.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp4.so")

# enums of include/fp4.h
FP4_OK = 0
FP4_ERR_INVALID_ARG = -1
FP4_ERR_UNSUPPORTED = -2
FP4_ERR_ALIGNMENT = -3
FP4_ERR_WORKSPACE = -4
FP4_ERR_HIP = -5
FP4_ERR_EXCHANGE = -6
FMT_MXFP4 = 0
FMT_NVFP4 = 1
FMT_MXINT4 = 2
FMT_NVINT4 = 3
DT_F32 = 0
DT_BF16 = 1
SCALES_ROWMAJOR = 0
SCALES_GEMM = 1
CODES_ROWMAJOR = 0
CODES_TILED = 1
GEMM_B_TILED = 0x100
GS_COMPUTE = 0
GS_GIVEN = 1
GS_COMPUTE_ONE_PASS = 2
SCALE_ABSMAX = 0
SCALE_MSE = 1
SCALE_FOUR_OVER_SIX = 2
ROUND_NEAREST = 0
ROUND_STOCHASTIC = 1
BLOCK = {FMT_MXFP4: 32, FMT_NVFP4: 16, FMT_MXINT4: 32, FMT_NVINT4: 16}
MX_FORMATS = (FMT_MXFP4, FMT_MXINT4)

EXPORTED = [
    "fp4_codes_bytes", "fp4_scales_bytes", "fp4_workspace_bytes", "fp4_scale_offset",
    "fp4_quantize", "fp4_quantize_noalloc", "fp4_quantize_one_pass_fits", "fp4_workspace_init",
    "fp4_global_scale",
    "fp4_quantize_batch_workspace_bytes", "fp4_quantize_batch", "fp4_dequantize",
    "fp4_error_workspace_bytes", "fp4_error_sums",
    "fp4_scales_to_gemm_layout", "fp4_gemm_workspace_bytes", "fp4_gemm",
    "fp4_gemm_w4a16_workspace_bytes", "fp4_gemm_w4a16", "fp4_status_str", "fp4_abi_version",
]


class FP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_str(status), status))


class QConfig(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("block", ctypes.c_int32), ("rotate", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("scale_layout", ctypes.c_int32),
                ("rounding", ctypes.c_int32), ("block_rows", ctypes.c_int32),
                ("rot_signs", ctypes.c_uint32 * 4), ("seed", ctypes.c_uint32 * 2),
                ("code_layout", ctypes.c_int32)]


class QuantJob(ctypes.Structure):
    """fp4_quant_job: the arguments of one fp4_quantize call (pointers as ints)."""
    _fields_ = [("cfg", QConfig), ("x", ctypes.c_void_p), ("xdt", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("gs_mode", ctypes.c_int32)]


def qconfig(fmt: int, rotate=False, scale_layout: int = SCALES_ROWMAJOR,
            rule: int = SCALE_ABSMAX, rounding: int = ROUND_NEAREST, block_rows: int = 1,
            signs: int = 0, seed=(0, 0), code_layout: int = CODES_ROWMAJOR) -> QConfig:
    """rotate: False / True (a rotation of the block size) or the rotation size
    (MX formats: 32, 64, 128).  signs: the rotation's sign mask as an integer
    (bit i negates element i of each group).  seed: stochastic-rounding key.
    code_layout: CODES_ROWMAJOR or CODES_TILED (8 KB tiles of 128 rows x 128
    elements, for weights the GEMM streams; rows and cols multiples of 128)."""
    G = BLOCK[fmt]
    rot = 0 if rotate is False or rotate is None else (G if rotate is True else int(rotate))
    q = QConfig(fmt, G, rot, rule, scale_layout, rounding, block_rows)
    for k in range(4):
        q.rot_signs[k] = (int(signs) >> (32 * k)) & 0xFFFFFFFF
    q.seed[0], q.seed[1] = int(seed[0]) & 0xFFFFFFFF, int(seed[1]) & 0xFFFFFFFF
    q.code_layout = code_layout
    return q


_lib = None


def lib():
    """Load libfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4.so is not built; run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        CP = ctypes.POINTER(QConfig)
        L.fp4_codes_bytes.restype = SZ
        L.fp4_codes_bytes.argtypes = [I64, I64]
        L.fp4_scales_bytes.restype = SZ
        L.fp4_scales_bytes.argtypes = [CP, I64, I64]
        L.fp4_workspace_bytes.restype = SZ
        L.fp4_workspace_bytes.argtypes = [CP, I64, I64]
        L.fp4_scale_offset.restype = I64
        L.fp4_scale_offset.argtypes = [CP, I64, I64, I64, I64]
        L.fp4_quantize.restype = ctypes.c_int
        L.fp4_quantize.argtypes = [CP, P, I32, I64, I64, I64, P, P, P, I32, P, SZ, P]
        L.fp4_quantize_noalloc.restype = ctypes.c_int
        L.fp4_quantize_noalloc.argtypes = [CP, P, I32, I64, I64, I64, P, P, P, I32, P]
        L.fp4_workspace_init.restype = ctypes.c_int
        L.fp4_workspace_init.argtypes = [P, SZ, P]
        L.fp4_quantize_one_pass_fits.restype = ctypes.c_int
        L.fp4_quantize_one_pass_fits.argtypes = [CP, I32, I64, I64, I64]
        L.fp4_global_scale.restype = ctypes.c_int
        L.fp4_global_scale.argtypes = [CP, P, I32, I64, I64, I64, P, P, SZ, P]
        L.fp4_quantize_batch_workspace_bytes.restype = SZ
        L.fp4_quantize_batch_workspace_bytes.argtypes = [I32]
        L.fp4_quantize_batch.restype = ctypes.c_int
        L.fp4_quantize_batch.argtypes = [I32, ctypes.POINTER(QuantJob), P, SZ, P]
        L.fp4_dequantize.restype = ctypes.c_int
        L.fp4_dequantize.argtypes = [CP, P, P, P, I64, I64, P, I32, I64, I32, P]
        L.fp4_error_workspace_bytes.restype = SZ
        L.fp4_error_workspace_bytes.argtypes = [CP, I64, I64]
        L.fp4_error_sums.restype = ctypes.c_int
        L.fp4_error_sums.argtypes = [CP, P, I32, I64, I64, I64, P, P, P, P, P, SZ, P]
        L.fp4_scales_to_gemm_layout.restype = ctypes.c_int
        L.fp4_scales_to_gemm_layout.argtypes = [CP, P, I64, I64, P, P]
        L.fp4_gemm_workspace_bytes.restype = SZ
        L.fp4_gemm_workspace_bytes.argtypes = [I32, I64, I64, I64]
        L.fp4_gemm.restype = ctypes.c_int
        L.fp4_gemm.argtypes = [I32, I64, I64, I64, P, P, P, P, P, P, P, I32, I64, P, SZ, P]
        L.fp4_gemm_w4a16_workspace_bytes.restype = SZ
        L.fp4_gemm_w4a16_workspace_bytes.argtypes = [I32, I64, I64, I64]
        L.fp4_gemm_w4a16.restype = ctypes.c_int
        L.fp4_gemm_w4a16.argtypes = [I32, I64, I64, I64, P, I64, P, P, P, P, I32, I64, P, SZ, P]
        L.fp4_status_str.restype = ctypes.c_char_p
        L.fp4_status_str.argtypes = [ctypes.c_int]
        L.fp4_abi_version.restype = ctypes.c_int
        L.fp4_abi_version.argtypes = []
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().fp4_status_str(int(status)).decode()


def _check(rc: int, what: str):
    if rc != FP4_OK:
        raise FP4Error(rc, what)


# ----------------------------------------------------------- raw ABI names
def fp4_codes_bytes(rows: int, cols: int) -> int:
    return lib().fp4_codes_bytes(rows, cols)


def fp4_scales_bytes(cfg: QConfig, rows: int, cols: int) -> int:
    return lib().fp4_scales_bytes(ctypes.byref(cfg), rows, cols)


def fp4_workspace_bytes(cfg: QConfig, rows: int, cols: int) -> int:
    return lib().fp4_workspace_bytes(ctypes.byref(cfg), rows, cols)


def fp4_scale_offset(cfg: QConfig, rows: int, cols: int, r: int, kb: int) -> int:
    return lib().fp4_scale_offset(ctypes.byref(cfg), rows, cols, r, kb)


def fp4_error_workspace_bytes(cfg: QConfig, rows: int, cols: int) -> int:
    return lib().fp4_error_workspace_bytes(ctypes.byref(cfg), rows, cols)


def fp4_gemm_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return lib().fp4_gemm_workspace_bytes(fmt, M, N, K)


def fp4_quantize(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode, ws,
                 ws_bytes, stream) -> int:
    """Raw call: pointers are ints (device addresses), stream an int handle."""
    return lib().fp4_quantize(ctypes.byref(cfg), x, xdt, rows, cols, ldx, codes, scales,
                              global_scale, gs_mode, ws, ws_bytes, stream)


def fp4_quantize_noalloc(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode,
                         stream) -> int:
    """Raw call: fp4_quantize with the library's static per-GPU scratch (no
    workspace argument, nothing allocated)."""
    return lib().fp4_quantize_noalloc(ctypes.byref(cfg), x, xdt, rows, cols, ldx, codes, scales,
                                      global_scale, gs_mode, stream)


def fp4_workspace_init(ws, ws_bytes, stream) -> int:
    return lib().fp4_workspace_init(ws, ws_bytes, stream)


def fp4_quantize_one_pass_fits(cfg, xdt, rows, cols, ldx) -> int:
    return lib().fp4_quantize_one_pass_fits(ctypes.byref(cfg), xdt, rows, cols, ldx)


def fp4_global_scale(cfg, x, xdt, rows, cols, ldx, global_scale, ws, ws_bytes, stream) -> int:
    return lib().fp4_global_scale(ctypes.byref(cfg), x, xdt, rows, cols, ldx, global_scale, ws,
                                  ws_bytes, stream)


def fp4_quantize_batch_workspace_bytes(n: int) -> int:
    return lib().fp4_quantize_batch_workspace_bytes(n)


def quant_job(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode) -> QuantJob:
    """One job for fp4_quantize_batch (pointers are ints, None for NULL)."""
    return QuantJob(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode)


def job_array(jobs):
    """A ctypes array of QuantJob for fp4_quantize_batch."""
    return (QuantJob * len(jobs))(*jobs)


def fp4_quantize_batch(n, jobs, ws, ws_bytes, stream) -> int:
    """Raw call: jobs is a ctypes array of QuantJob (job_array) or None."""
    return lib().fp4_quantize_batch(n, jobs, ws, ws_bytes, stream)


def fp4_dequantize(cfg, codes, scales, global_scale, rows, cols, y, ydt, ldy, inverse_rotate,
                   stream) -> int:
    return lib().fp4_dequantize(ctypes.byref(cfg), codes, scales, global_scale, rows, cols, y,
                                ydt, ldy, inverse_rotate, stream)


def fp4_error_sums(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, sums, ws,
                   ws_bytes, stream) -> int:
    return lib().fp4_error_sums(ctypes.byref(cfg), x, xdt, rows, cols, ldx, codes, scales,
                                global_scale, sums, ws, ws_bytes, stream)


def fp4_scales_to_gemm_layout(cfg, rowmajor, rows, cols, gemm_scales, stream) -> int:
    return lib().fp4_scales_to_gemm_layout(ctypes.byref(cfg), rowmajor, rows, cols, gemm_scales,
                                           stream)


def fp4_gemm(fmt, M, N, K, a_codes, a_scales, a_gs, b_codes, b_scales, b_gs, y, ydt, ldy, ws,
             ws_bytes, stream) -> int:
    return lib().fp4_gemm(fmt, M, N, K, a_codes, a_scales, a_gs, b_codes, b_scales, b_gs, y, ydt,
                          ldy, ws, ws_bytes, stream)


def fp4_gemm_w4a16_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return lib().fp4_gemm_w4a16_workspace_bytes(fmt, M, N, K)


def fp4_gemm_w4a16(fmt, M, N, K, a, lda, b_codes, b_scales, b_gs, y, ydt, ldy, ws, ws_bytes,
                   stream) -> int:
    return lib().fp4_gemm_w4a16(fmt, M, N, K, a, lda, b_codes, b_scales, b_gs, y, ydt, ldy, ws,
                                ws_bytes, stream)


# ----------------------------------------------------------- torch helpers
def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError("x must be float32 or bfloat16, got %s" % t.dtype)


_ws_cache: dict = {}


def _scratch_workspace(nbytes: int, device, stream: int):
    """Scratch of the NVFP4 global-amax pass (partial maxima) and of the
    single-pass exchange region (zero when allocated, left ready by every
    call), one per (device, stream, size).  Calls on one stream are ordered,
    so they never overlap on their buffer; calls on two streams get two
    buffers (a shared one would mix the partial maxima or the exchange slots
    of concurrent calls)."""
    torch = _torch()
    key = (str(device), int(stream or 0), nbytes)
    t = _ws_cache.get(key)
    if t is None:
        t = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        _ws_cache[key] = t
    return t


# Word 1 of the single-pass exchange region (byte 4096 + 4 of the NVFP4
# workspace): non-zero after a call whose grid-wide wait gave up.
EXCHANGE_FLAG_OFFSET = 4096 + 4


def one_pass_gave_up(flag_word: int, global_scale: float) -> bool:
    """True when a single-pass call's exchange wait gave up: the kernel sets
    the exchange region's flag word and writes NaN as the tensor scale."""
    return int(flag_word) != 0 or global_scale != global_scale


_gemm_ws_cache = {}


def _gemm_workspace(nbytes: int, device, stream: int):
    """GEMM split-K workspace (fp32 partial sums; any contents) per (device,
    stream), grown to the largest size asked for: calls on one stream never
    overlap on it."""
    torch = _torch()
    key = (str(device), int(stream or 0))
    t = _gemm_ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        _gemm_ws_cache[key] = t
    return t


def gemm_workspace(nbytes: int, device):
    """A fresh GEMM workspace of nbytes (for callers that keep their own, e.g.
    one per stream or per captured graph)."""
    torch = _torch()
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def _workspace_arg(workspace, device, what: str):
    """(pointer, size in bytes) of a caller's workspace tensor: the size passed
    to the C ABI is the buffer's own, so that a buffer smaller than the call
    needs makes the library run without it instead of writing past it."""
    torch = _torch()
    if workspace is None:
        return None, 0
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("%s: workspace must be a contiguous uint8 tensor" % what)
    if workspace.device != device:
        raise ValueError("%s: workspace on %s, operands on %s" % (what, workspace.device, device))
    return workspace.data_ptr(), workspace.numel()


def _check_out(out, M: int, N: int, device, what: str):
    """The output of a product: an [M, N] fp32 / bf16 tensor on the operands'
    device with unit stride along N (its row stride becomes ldy)."""
    torch = _torch()
    if out.dim() != 2 or tuple(out.shape) != (M, N):
        raise ValueError("%s: out must be [%d, %d], got %s" % (what, M, N, tuple(out.shape)))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("%s: out must be float32 or bfloat16, got %s" % (what, out.dtype))
    if N > 1 and out.stride(1) != 1:
        raise ValueError("%s: out needs unit stride along N" % what)
    if M > 1 and out.stride(0) < N:
        raise ValueError("%s: out rows overlap (stride %d < N)" % (what, out.stride(0)))
    if out.device != device:
        raise ValueError("%s: out on %s, operands on %s" % (what, out.device, device))


def _same_rotation(a: QConfig, b: QConfig) -> bool:
    return a.rotate == b.rotate and list(a.rot_signs) == list(b.rot_signs)


def check_gemm_operands(a: "Quantized", b: "Quantized"):
    """Operand checks of gemm(): same format and K, GEMM-layout scales for the
    MX formats, and the same rotation (size and sign diagonal) on both sides:
    the product of two differently rotated operands is not A B^T."""
    fa, fb = a.cfg.fmt, b.cfg.fmt
    if fa != fb:
        raise ValueError("gemm: operand formats differ (%d, %d)" % (fa, fb))
    if a.cols != b.cols:
        raise ValueError("gemm: K differs (%d, %d)" % (a.cols, b.cols))
    if fa in MX_FORMATS and (a.cfg.scale_layout != SCALES_GEMM or b.cfg.scale_layout != SCALES_GEMM):
        raise ValueError("gemm: MX operands need FP4_SCALES_GEMM scales")
    if a.cfg.code_layout != CODES_ROWMAJOR:
        raise ValueError("gemm: A codes must be row-major (only B may be tiled)")
    if not _same_rotation(a.cfg, b.cfg):
        raise ValueError("gemm: operands quantized with different rotations")


@dataclass
class Quantized:
    """Packed FP4 tensor: codes [rows, cols/2] u8, scales (layout of cfg) u8,
    global_scale float32[1] (NVFP4) and the configuration."""
    codes: object
    scales: object
    global_scale: object
    cfg: QConfig
    rows: int
    cols: int


def quantize(x, fmt: int, rotate=False, scale_layout: int = SCALES_ROWMAJOR,
             global_scale=None, out: Quantized | None = None,
             rule: int = SCALE_ABSMAX, rounding: int = ROUND_NEAREST, block_rows: int = 1,
             signs: int = 0, seed=(0, 0), one_pass: bool = False,
             check_one_pass: bool = False, code_layout: int = CODES_ROWMAJOR) -> Quantized:
    """Quantize a 2-D CUDA tensor (fp32 or bf16, unit stride along the last
    axis).  NVFP4: ``global_scale`` (a float32[1] CUDA tensor) is used as given
    when passed, otherwise computed from the tensor's amax (``one_pass``: the
    amax and the encoding in one launch when the tensor fits, the same
    results).  ``rule`` selects the block-scale rule (SCALE_ABSMAX, SCALE_MSE,
    SCALE_FOUR_OVER_SIX).  ``code_layout``: CODES_TILED writes the codes in
    8 KB tiles of 128 rows x 128 elements (weights for gemm / gemm_w4a16 as
    their B operand; rows and cols multiples of 128).

    ``check_one_pass`` (with ``one_pass``): synchronise the stream and raise
    FP4Error(FP4_ERR_EXCHANGE) when the single launch's grid-wide wait gave up
    (its workgroups were not all resident, e.g. another grid-synchronising
    kernel held CUs); the workspace's exchange region is re-zeroed first, so
    the next call starts clean.  The workspace is per stream: single-pass
    calls on different streams must still not run at the same time."""
    torch = _torch()
    assert x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    cfg = qconfig(fmt, rotate, scale_layout, rule, rounding, block_rows, signs, seed, code_layout)
    if out is None:
        codes = torch.empty(max(fp4_codes_bytes(rows, cols), 16), dtype=torch.uint8, device=x.device)
        scales = torch.empty(max(fp4_scales_bytes(cfg, rows, cols), 16), dtype=torch.uint8,
                             device=x.device)
        gs = torch.zeros(1, dtype=torch.float32, device=x.device)
        out = Quantized(codes, scales, gs, cfg, rows, cols)
    gs_mode = GS_COMPUTE_ONE_PASS if one_pass else GS_COMPUTE
    if fmt not in MX_FORMATS and global_scale is not None:
        out.global_scale.copy_(global_scale.reshape(1))
        gs_mode = GS_GIVEN
    stream = _stream()
    wsb = fp4_workspace_bytes(cfg, rows, cols)
    ws = _scratch_workspace(wsb, x.device, stream) if wsb else None
    rc = fp4_quantize(cfg, x.data_ptr(), _dt(x), rows, cols, x.stride(0), out.codes.data_ptr(),
                      out.scales.data_ptr(), out.global_scale.data_ptr(), gs_mode, _ptr(ws), wsb,
                      stream)
    _check(rc, "fp4_quantize")
    if check_one_pass and gs_mode == GS_COMPUTE_ONE_PASS and ws is not None:
        torch.cuda.current_stream().synchronize()
        off = EXCHANGE_FLAG_OFFSET
        flag = int(ws[off:off + 4].view(torch.int32).item())
        if one_pass_gave_up(flag, float(out.global_scale.item())):
            _check(fp4_workspace_init(ws.data_ptr(), wsb, stream), "fp4_workspace_init")
            torch.cuda.current_stream().synchronize()
            raise FP4Error(FP4_ERR_EXCHANGE, "fp4_quantize (single pass)")
    return out


def quantize_batch(items: list) -> list:
    """Several quantizations in one fp4_quantize_batch call.  items: dicts
    with the arguments of quantize() ("x" and "fmt", optionally "rotate",
    "scale_layout", "global_scale", "rule", "rounding", "block_rows",
    "signs", "seed", "code_layout", "out").  Returns one Quantized per item, the same as
    quantize() would give."""
    torch = _torch()
    outs, jobs = [], []
    dev = None
    for it in items:
        x, fmt = it["x"], it["fmt"]
        assert x.dim() == 2 and x.stride(1) == 1
        dev = x.device
        rows, cols = x.shape
        cfg = qconfig(fmt, it.get("rotate", False), it.get("scale_layout", SCALES_ROWMAJOR),
                      it.get("rule", SCALE_ABSMAX), it.get("rounding", ROUND_NEAREST),
                      it.get("block_rows", 1), it.get("signs", 0), it.get("seed", (0, 0)),
                      it.get("code_layout", CODES_ROWMAJOR))
        out = it.get("out")
        if out is None:
            codes = torch.empty(max(fp4_codes_bytes(rows, cols), 16), dtype=torch.uint8, device=dev)
            scales = torch.empty(max(fp4_scales_bytes(cfg, rows, cols), 16), dtype=torch.uint8,
                                 device=dev)
            out = Quantized(codes, scales, torch.zeros(1, dtype=torch.float32, device=dev), cfg,
                            rows, cols)
        gs_mode = GS_COMPUTE
        if fmt not in MX_FORMATS and it.get("global_scale") is not None:
            out.global_scale.copy_(it["global_scale"].reshape(1))
            gs_mode = GS_GIVEN
        outs.append(out)
        jobs.append(quant_job(cfg, x.data_ptr(), _dt(x), rows, cols, x.stride(0),
                              out.codes.data_ptr(), out.scales.data_ptr(),
                              out.global_scale.data_ptr(), gs_mode))
    if not jobs:
        return outs
    wsb = fp4_quantize_batch_workspace_bytes(len(jobs))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    rc = fp4_quantize_batch(len(jobs), job_array(jobs), ws.data_ptr(), wsb, _stream())
    _check(rc, "fp4_quantize_batch")
    return outs


def global_scale(x, rotate=False, out=None, fmt: int = FMT_NVFP4, signs: int = 0):
    """NVFP4 (or NVINT4) per-tensor scale of a 2-D CUDA tensor (float32[1]
    CUDA tensor)."""
    torch = _torch()
    rows, cols = x.shape
    cfg = qconfig(fmt, rotate, signs=signs)
    if out is None:
        out = torch.zeros(1, dtype=torch.float32, device=x.device)
    stream = _stream()
    wsb = fp4_workspace_bytes(cfg, rows, cols)
    ws = _scratch_workspace(wsb, x.device, stream)
    rc = fp4_global_scale(cfg, x.data_ptr(), _dt(x), rows, cols, x.stride(0), out.data_ptr(),
                          ws.data_ptr(), wsb, stream)
    _check(rc, "fp4_global_scale")
    return out


def codes_view(q: Quantized):
    """The codes as [rows, cols/2] bytes (row-major codes only)."""
    if q.cfg.code_layout != CODES_ROWMAJOR:
        raise ValueError("codes_view: the codes are tiled")
    return q.codes[: q.rows * q.cols // 2].view(q.rows, q.cols // 2)


def dequantize(q: Quantized, dtype=None, inverse_rotate: bool = False):
    torch = _torch()
    dtype = dtype or torch.float32
    y = torch.empty(q.rows, q.cols, dtype=dtype, device=q.codes.device)
    rc = fp4_dequantize(q.cfg, q.codes.data_ptr(), q.scales.data_ptr(), q.global_scale.data_ptr(),
                        q.rows, q.cols, y.data_ptr(), _dt(y), y.stride(0), int(inverse_rotate),
                        _stream())
    _check(rc, "fp4_dequantize")
    return y


def error_sums(x, q: Quantized):
    """[sum (x-x^)^2, sum x^2, sum x x^, sum x^^2] (float64 CUDA tensor)."""
    torch = _torch()
    rows, cols = x.shape
    wsb = fp4_error_workspace_bytes(q.cfg, rows, cols)
    ws = torch.empty(max(wsb, 64), dtype=torch.uint8, device=x.device)
    sums = torch.empty(4, dtype=torch.float64, device=x.device)
    rc = fp4_error_sums(q.cfg, x.data_ptr(), _dt(x), rows, cols, x.stride(0), q.codes.data_ptr(),
                        q.scales.data_ptr(), q.global_scale.data_ptr(), sums.data_ptr(),
                        ws.data_ptr(), wsb, _stream())
    _check(rc, "fp4_error_sums")
    return sums


def scales_to_gemm_layout(rowmajor, rows: int, cols: int, fmt: int = FMT_MXFP4):
    torch = _torch()
    cfg = qconfig(fmt, False, SCALES_GEMM)
    out = torch.empty(max(fp4_scales_bytes(cfg, rows, cols), 16), dtype=torch.uint8,
                      device=rowmajor.device)
    rc = fp4_scales_to_gemm_layout(cfg, rowmajor.data_ptr(), rows, cols, out.data_ptr(), _stream())
    _check(rc, "fp4_scales_to_gemm_layout")
    return out


def gemm_w4a16(a, b: Quantized, out_dtype=None, out=None, workspace=None):
    """Y = A * dequant(B)^T for bf16 activations A [M, K] (unit stride along K)
    and quantized weights B (scales in GEMM layout).  ``workspace``: a uint8
    tensor on A's device (its whole size is offered; one smaller than
    fp4_gemm_w4a16_workspace_bytes() makes the call run without split-K)."""
    torch = _torch()
    if a.dim() != 2 or a.stride(1) != 1 or a.dtype != torch.bfloat16:
        raise ValueError("gemm_w4a16: A must be a 2-D bf16 tensor with unit stride along K")
    M, K = a.shape
    fmt, N = b.cfg.fmt, b.rows
    if b.cols != K:
        raise ValueError("gemm_w4a16: K differs (%d, %d)" % (K, b.cols))
    if fmt in MX_FORMATS and b.cfg.scale_layout != SCALES_GEMM:
        raise ValueError("gemm_w4a16: MX weights need FP4_SCALES_GEMM scales")
    if b.cfg.code_layout == CODES_TILED:
        fmt |= GEMM_B_TILED
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype or torch.bfloat16, device=a.device)
    _check_out(out, M, N, a.device, "gemm_w4a16")
    stream = _stream()
    if workspace is None:
        wsb = fp4_gemm_w4a16_workspace_bytes(fmt, M, N, K)
        workspace = _gemm_workspace(wsb, a.device, stream) if wsb else None
    ws_ptr, ws_bytes = _workspace_arg(workspace, a.device, "gemm_w4a16")
    rc = fp4_gemm_w4a16(fmt, M, N, K, a.data_ptr(), a.stride(0), b.codes.data_ptr(),
                        b.scales.data_ptr(), b.global_scale.data_ptr(), out.data_ptr(), _dt(out),
                        out.stride(0), ws_ptr, ws_bytes, stream)
    _check(rc, "fp4_gemm_w4a16")
    return out


def gemm(a: Quantized, b: Quantized, out_dtype=None, out=None, workspace=None):
    """Y = A * B^T for two quantized operands sharing K, format and rotation
    (MX scales in GEMM layout).  ``workspace``: a uint8 tensor on the operands'
    device (its whole size is offered; one smaller than
    fp4_gemm_workspace_bytes() makes the call run without split-K)."""
    torch = _torch()
    check_gemm_operands(a, b)
    fmt = a.cfg.fmt | (GEMM_B_TILED if b.cfg.code_layout == CODES_TILED else 0)
    M, N, K = a.rows, b.rows, a.cols
    device = a.codes.device
    if b.codes.device != device:
        raise ValueError("gemm: operands on %s and %s" % (device, b.codes.device))
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype or torch.bfloat16, device=device)
    _check_out(out, M, N, device, "gemm")
    stream = _stream()
    if workspace is None:
        wsb = fp4_gemm_workspace_bytes(fmt, M, N, K)
        workspace = _gemm_workspace(wsb, device, stream) if wsb else None
    ws_ptr, ws_bytes = _workspace_arg(workspace, device, "gemm")
    rc = fp4_gemm(fmt, M, N, K, a.codes.data_ptr(), a.scales.data_ptr(),
                  a.global_scale.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
                  b.global_scale.data_ptr(), out.data_ptr(), _dt(out), out.stride(0),
                  ws_ptr, ws_bytes, stream)
    _check(rc, "fp4_gemm")
    return out

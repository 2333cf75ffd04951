"""CPU oracle for block-wise microscaling FP4 (MXFP4 / NVFP4) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never loads it, and the two share no code.

The arithmetic lives in ``fp4_oracle.c`` (plain C, IEEE binary32/binary64, no
FMA contraction); this module only marshals numpy arrays into it through ctypes.
Every function of the C file cites the passage it follows.

Pinning status: every function here is pinned by ``tests/test_oracle_pins.py``
(worked examples and printed emulation results of "NVFP4 vs MXFP4: 4-Bit
Floating Point for LLM Training and Inference (2026)", format definitions,
closed forms, brute force on tiny inputs, invariants).  No function is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

class QSpec(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("rot_n", ctypes.c_int), ("signs", ctypes.c_uint32 * 4),
                ("rule", ctypes.c_int), ("rounding", ctypes.c_int), ("seed", ctypes.c_uint32 * 2),
                ("block_rows", ctypes.c_int)]


MXFP4 = 0
NVFP4 = 1
MXINT4 = 2
NVINT4 = 3
BLOCK = {MXFP4: 32, NVFP4: 16, MXINT4: 32, NVINT4: 16}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no vectorisation tricks)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    l = ctypes.c_long
    L.ora_e2m1_decode.restype = ctypes.c_double
    L.ora_e2m1_decode.argtypes = [ctypes.c_int]
    L.ora_e2m1_encode.restype = ctypes.c_int
    L.ora_e2m1_encode.argtypes = [ctypes.c_float]
    L.ora_e4m3_decode.restype = ctypes.c_double
    L.ora_e4m3_decode.argtypes = [ctypes.c_int]
    L.ora_e4m3_encode.restype = ctypes.c_int
    L.ora_e4m3_encode.argtypes = [ctypes.c_float]
    L.ora_e8m0_decode.restype = ctypes.c_double
    L.ora_e8m0_decode.argtypes = [ctypes.c_int]
    L.ora_rotate.restype = ctypes.c_int
    L.ora_rotate.argtypes = [P, P, l, l, ctypes.c_int]
    L.ora_quantize.restype = ctypes.c_int
    L.ora_quantize.argtypes = [ctypes.c_int, ctypes.c_int, P, l, l, P, P, P, ctypes.c_int]
    L.ora_quantize_rule.restype = ctypes.c_int
    L.ora_quantize_rule.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, l, l, P, P, P,
                                    ctypes.c_int]
    L.ora_quantize_spec.restype = ctypes.c_int
    L.ora_quantize_spec.argtypes = [ctypes.POINTER(QSpec), P, l, l, P, P, P, ctypes.c_int]
    L.ora_tensor_scale.restype = ctypes.c_int
    L.ora_tensor_scale.argtypes = [ctypes.c_int, ctypes.c_int, P, P, l, l, P]
    L.ora_dequantize_rot.restype = ctypes.c_int
    L.ora_dequantize_rot.argtypes = [ctypes.c_int, P, P, ctypes.c_float, l, l, ctypes.c_int, P, P]
    L.ora_rotate_signed.restype = ctypes.c_int
    L.ora_rotate_signed.argtypes = [P, P, l, l, ctypes.c_int, P, ctypes.c_int]
    L.ora_philox4x32_10.restype = None
    L.ora_philox4x32_10.argtypes = [P, P, P]
    L.ora_e2m1_encode_sr.restype = ctypes.c_int
    L.ora_e2m1_encode_sr.argtypes = [ctypes.c_float, ctypes.c_double]
    L.ora_dequantize.restype = ctypes.c_int
    L.ora_dequantize.argtypes = [ctypes.c_int, P, P, ctypes.c_float, l, l, ctypes.c_int, P]
    L.ora_error_sums.restype = None
    L.ora_error_sums.argtypes = [P, P, l, P]
    L.ora_gemm_entries.restype = ctypes.c_int
    L.ora_gemm_entries.argtypes = [ctypes.c_int, l, P, P, ctypes.c_float, P, P,
                                   ctypes.c_float, l, P, P, P, P]
    L.ora_gemm_w4a16_entries.restype = ctypes.c_int
    L.ora_gemm_w4a16_entries.argtypes = [ctypes.c_int, l, P, l, P, P, ctypes.c_float, l, P, P,
                                         P, P]
    L.ora_e2m1_encode_array.restype = None
    L.ora_e2m1_encode_array.argtypes = [P, l, P]
    L.ora_int4_decode.restype = ctypes.c_double
    L.ora_int4_decode.argtypes = [ctypes.c_int]
    L.ora_int4_encode.restype = ctypes.c_int
    L.ora_int4_encode.argtypes = [ctypes.c_float]
    L.ora_int4_encode_array.restype = None
    L.ora_int4_encode_array.argtypes = [P, l, P]
    L.ora_e4m3_encode_array.restype = None
    L.ora_e4m3_encode_array.argtypes = [P, l, P]
    L.ora_tile_codes.restype = ctypes.c_int
    L.ora_tile_codes.argtypes = [P, l, l, P]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _load(_LIB)
    return _lib


def use_library(path: str | None):
    """Point the wrapper at another build of the oracle source (the mutation
    test loads deliberately broken copies); None restores the default."""
    global _lib
    _lib = None if path is None else _load(path)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def e2m1_decode(code: int) -> float:
    return lib().ora_e2m1_decode(int(code))


def e2m1_encode(q: float) -> int:
    return lib().ora_e2m1_encode(float(q))


def e2m1_encode_array(q) -> np.ndarray:
    q = _f32(q).reshape(-1)
    out = np.empty(q.size, dtype=np.uint8)
    lib().ora_e2m1_encode_array(_p(q), q.size, _p(out))
    return out


def int4_decode(code: int) -> float:
    return lib().ora_int4_decode(int(code))


def int4_encode(q: float) -> int:
    return lib().ora_int4_encode(float(q))


def int4_encode_array(q) -> np.ndarray:
    q = _f32(q).reshape(-1)
    out = np.empty(q.size, dtype=np.uint8)
    lib().ora_int4_encode_array(_p(q), q.size, _p(out))
    return out


def e4m3_decode(code: int) -> float:
    return lib().ora_e4m3_decode(int(code))


def e4m3_encode(t: float) -> int:
    return lib().ora_e4m3_encode(float(t))


def e4m3_encode_array(t) -> np.ndarray:
    t = _f32(t).reshape(-1)
    out = np.empty(t.size, dtype=np.uint8)
    lib().ora_e4m3_encode_array(_p(t), t.size, _p(out))
    return out


def e8m0_decode(code: int) -> float:
    return lib().ora_e8m0_decode(int(code))


def rotate(x, n: int) -> np.ndarray:
    """Block Hadamard (Sylvester, / sqrt(n)) along the last axis."""
    x = _f32(x)
    rows, cols = (1, x.size) if x.ndim == 1 else x.shape
    y = np.empty_like(x)
    rc = lib().ora_rotate(_p(x), _p(y), rows, cols, n)
    if rc != 0:
        raise ValueError("ora_rotate: bad arguments")
    return y


SCALE_ABSMAX = 0
SCALE_MSE = 1
SCALE_FOUR_OVER_SIX = 2
ROUND_NEAREST = 0
ROUND_STOCHASTIC = 1


def _signs_array(signs) -> np.ndarray:
    """Sign mask of a rotation group as four uint32 words (bit i: element i
    negated); accepts None, an int (up to 128 bits) or four words."""
    if signs is None:
        return np.zeros(4, dtype=np.uint32)
    if isinstance(signs, (int, np.integer)):
        v = int(signs)
        return np.array([(v >> (32 * k)) & 0xFFFFFFFF for k in range(4)], dtype=np.uint32)
    return np.ascontiguousarray(signs, dtype=np.uint32).reshape(4)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(4)
    k = np.ascontiguousarray(key, dtype=np.uint32).reshape(2)
    out = np.zeros(4, dtype=np.uint32)
    lib().ora_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def e2m1_encode_sr(q: float, u: float) -> int:
    return lib().ora_e2m1_encode_sr(float(q), float(u))


def rotate_signed(x, n: int, signs=None, inverse: bool = False) -> np.ndarray:
    x = _f32(x)
    rows, cols = (1, x.size) if x.ndim == 1 else x.shape
    y = np.empty_like(x)
    sg = _signs_array(signs)
    rc = lib().ora_rotate_signed(_p(x), _p(y), rows, cols, int(n), _p(sg), int(bool(inverse)))
    if rc != 0:
        raise ValueError("ora_rotate_signed: bad arguments")
    return y


def quantize_spec(x, fmt: int, rot_n: int = 0, signs=None, rule: int = SCALE_ABSMAX,
                  rounding: int = ROUND_NEAREST, seed=(0, 0), block_rows: int = 1,
                  ts: float | None = None):
    """The general quantizer: rotation of size rot_n (0, the block size, or 64 /
    128 for MX formats) with a sign mask, scale rule, nearest or stochastic
    rounding (Philox4x32-10 keyed by seed), NVFP4 16x16 blocks.  Returns
    (codes, scales, ts)."""
    x = _f32(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, cols = x.shape
    G = BLOCK[fmt]
    q = QSpec()
    q.fmt, q.rot_n, q.rule, q.rounding, q.block_rows = fmt, int(rot_n), int(rule), int(rounding), int(block_rows)
    sg = _signs_array(signs)
    for k in range(4):
        q.signs[k] = int(sg[k])
    q.seed[0], q.seed[1] = int(seed[0]) & 0xFFFFFFFF, int(seed[1]) & 0xFFFFFFFF
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // G), dtype=np.uint8)
    tsa = np.zeros(1, dtype=np.float32)
    if ts is not None:
        tsa[0] = ts
    rc = lib().ora_quantize_spec(ctypes.byref(q), _p(x), rows, cols, _p(codes), _p(scales), _p(tsa),
                                 int(ts is not None))
    if rc != 0:
        raise ValueError("ora_quantize_spec: bad arguments")
    return codes, scales, np.float32(tsa[0])


def tensor_scale(x, fmt: int, rotate: bool = False, signs=None) -> np.float32:
    """NV per-tensor scale of x (rotated by the block size when rotate), the
    same number quantize() computes: amax / 2688 (NVFP4) or / 3136 (NVINT4)."""
    x = _f32(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, cols = x.shape
    sg = _signs_array(signs)
    ts = np.zeros(1, dtype=np.float32)
    rc = lib().ora_tensor_scale(fmt, BLOCK[fmt] if rotate else 0, _p(sg), _p(x), rows, cols, _p(ts))
    if rc != 0:
        raise ValueError("ora_tensor_scale: bad arguments")
    return np.float32(ts[0])


def dequantize_rot(codes, scales, fmt: int, ts: float = 0.0, rot_n: int = 0, signs=None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    y = np.empty((rows, cols), dtype=np.float32)
    sg = _signs_array(signs)
    rc = lib().ora_dequantize_rot(fmt, _p(codes), _p(scales), float(ts), rows, cols, int(rot_n),
                                  _p(sg), _p(y))
    if rc != 0:
        raise ValueError("ora_dequantize_rot: bad arguments")
    return y


def quantize(x, fmt: int, rotate: bool = False, ts: float | None = None, rule: int = SCALE_ABSMAX):
    """Returns (codes [rows, cols/2] u8, scales [rows, cols/G] u8, ts float32).
    rule: SCALE_ABSMAX, SCALE_MSE (windowed squared-error search over the
    block-scale code) or SCALE_FOUR_OVER_SIX (NVFP4: maximum onto 6 or 4)."""
    x = _f32(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, cols = x.shape
    G = BLOCK[fmt]
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // G), dtype=np.uint8)
    tsa = np.zeros(1, dtype=np.float32)
    if ts is not None:
        tsa[0] = ts
    rc = lib().ora_quantize_rule(fmt, int(bool(rotate)), int(rule), _p(x), rows, cols, _p(codes),
                                 _p(scales), _p(tsa), int(ts is not None))
    if rc != 0:
        raise ValueError("ora_quantize_rule: bad arguments")
    return codes, scales, np.float32(tsa[0])


def dequantize(codes, scales, fmt: int, ts: float = 0.0, inverse_rotate: bool = False):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    y = np.empty((rows, cols), dtype=np.float32)
    rc = lib().ora_dequantize(fmt, _p(codes), _p(scales), float(ts), rows, cols,
                              int(bool(inverse_rotate)), _p(y))
    if rc != 0:
        raise ValueError("ora_dequantize: bad arguments")
    return y


def tile_codes(codes) -> np.ndarray:
    """Row-major packed codes [rows, row_bytes] (rows % 128 == 0, row_bytes %
    64 == 0) in the library's tiled code layout (8 KB tiles of 128 rows x 64
    bytes; see ora_tile_codes), as a flat byte array."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, row_bytes = codes.shape
    out = np.zeros(rows * row_bytes, dtype=np.uint8)
    if lib().ora_tile_codes(_p(codes), rows, row_bytes, _p(out)) != 0:
        raise ValueError("ora_tile_codes: rows must be a multiple of 128, row bytes of 64")
    return out


def error_sums(x, xhat) -> np.ndarray:
    """[sum (x-x^)^2, sum x^2, sum x x^, sum x^^2] in double."""
    x = _f32(x).reshape(-1)
    xhat = _f32(xhat).reshape(-1)
    assert x.size == xhat.size
    out = np.zeros(4, dtype=np.float64)
    lib().ora_error_sums(_p(x), _p(xhat), x.size, _p(out))
    return out


def nmse(x, xhat) -> float:
    s = error_sums(x, xhat)
    return float(s[0] / s[1])


def cosine(x, xhat) -> float:
    s = error_sums(x, xhat)
    return float(s[2] / np.sqrt(s[1] * s[3]))


def host_threads() -> int:
    """Threads for the entry-wise products: the host's cores (at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _over_chunks(n: int, K: int, run):
    """run(lo, hi) over contiguous chunks of n entries, on host threads when the
    work is large (each entry is computed on its own, so the results do not
    depend on the split; the C calls release the interpreter lock)."""
    workers = host_threads()
    if n * max(K, 1) < (1 << 24) or workers == 1 or n < 2 * workers:
        return [run(0, n)]
    from concurrent.futures import ThreadPoolExecutor
    step = (n + 4 * workers - 1) // (4 * workers)
    spans = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda sp: run(*sp), spans))


def gemm_entries(fmt: int, K: int, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts,
                 rows, cols):
    """(y, |A||B|) at the listed (row, col) pairs of Y = A B^T, in double."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.size == cols.size
    y = np.zeros(rows.size, dtype=np.float64)
    ab = np.zeros(rows.size, dtype=np.float64)

    def run(lo, hi):
        return lib().ora_gemm_entries(fmt, K, _p(a_codes), _p(a_scales), float(a_ts), _p(b_codes),
                                      _p(b_scales), float(b_ts), hi - lo, _p(rows[lo:hi]),
                                      _p(cols[lo:hi]), _p(y[lo:hi]), _p(ab[lo:hi]))

    if any(rc != 0 for rc in _over_chunks(rows.size, K, run)):
        raise ValueError("ora_gemm_entries: bad arguments")
    return y, ab


def gemm_w4a16_entries(fmt: int, K: int, a, b_codes, b_scales, b_ts, rows, cols):
    """(y, |A||B|) of the weight-only product Y = A dequant(B)^T at the listed
    (row, col) pairs, in double; a is the [M, K] activation array (fp32 values)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.size == cols.size and a.ndim == 2 and a.shape[1] == K
    y = np.zeros(rows.size, dtype=np.float64)
    ab = np.zeros(rows.size, dtype=np.float64)

    def run(lo, hi):
        return lib().ora_gemm_w4a16_entries(fmt, K, _p(a), K, _p(b_codes), _p(b_scales),
                                            float(b_ts), hi - lo, _p(rows[lo:hi]),
                                            _p(cols[lo:hi]), _p(y[lo:hi]), _p(ab[lo:hi]))

    if any(rc != 0 for rc in _over_chunks(rows.size, K, run)):
        raise ValueError("ora_gemm_w4a16_entries: bad arguments")
    return y, ab


def gemm_w4a16_full(fmt: int, K: int, a, b_codes, b_scales, b_ts):
    M = a.shape[0]
    N = b_codes.shape[0]
    r, c = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, ab = gemm_w4a16_entries(fmt, K, a, b_codes, b_scales, b_ts, r.reshape(-1), c.reshape(-1))
    return y.reshape(M, N), ab.reshape(M, N)


def gemm_full(fmt: int, K: int, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts):
    M = a_codes.shape[0]
    N = b_codes.shape[0]
    r, c = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, ab = gemm_entries(fmt, K, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts,
                         r.reshape(-1), c.reshape(-1))
    return y.reshape(M, N), ab.reshape(M, N)

"""Seeded synthetic inputs for the FP4 microscaling workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers and shapes them into tensors; it holds
none of the quantization arithmetic (no rounding onto a grid, no scales, no
rotation).

Random source: numpy's PCG64 bit generator seeded through ``SeedSequence([seed,
stream])``; uniform doubles are ``(next_uint64 >> 11) * 2**-53``.  The shaping
transforms are written out here so that they do not depend on numpy's own
distribution algorithms:

* Laplace(0, b) by inverse CDF: ``x = -b * sgn(u) * ln(1 - 2|u|)``, u uniform in
  (-1/2, 1/2).
* Normal(0, s^2) by Box-Muller in double.
* Outlier subsets (a fraction of entries, or k channels) are the k positions with
  the smallest of n fresh uniforms, i.e. a uniformly random k-subset without
  replacement.
* bf16 is fp32 rounded to nearest-even on the upper 16 bits.

The workloads mirror the pages' synthetic tensors: heavy-tailed 131,072-element
tensors with 1 % outliers ("Portable FP4 Quantization for Heterogeneous
Accelerators", section 3.1), and Llama-shaped activations (Laplace-like, with a
few outlier channels) and weights (Gaussian) as in "Bridging the Gap Between
Promise and Performance for Microscaling FP4 Quantization", section 3 and
Figure 5.  No model weights or datasets are used.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "uniform_open", "laplace", "normal", "choose_subset", "to_bf16_bits",
    "bf16_bits_to_f32", "scale_entries", "scale_columns", "CONFIGS",
    "cfg1_tensor", "cfg2_tensor", "cfg3_tensor", "gemm_activation", "gemm_weight",
    "random_codes", "random_scales", "edge_tensor", "extreme_scales",
]


def rng(seed: int, stream: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def uniform_open(g: np.random.Generator, n: int) -> np.ndarray:
    """n uniform doubles in the open interval (0, 1)."""
    u = g.random(n)
    u[u == 0.0] = 2.0 ** -54
    return u


def laplace(g: np.random.Generator, n: int, b: float) -> np.ndarray:
    u = uniform_open(g, n) - 0.5
    return -b * np.sign(u) * np.log1p(-2.0 * np.abs(u))


def normal(g: np.random.Generator, n: int, std: float) -> np.ndarray:
    m = (n + 1) // 2
    u1 = uniform_open(g, m)
    u2 = g.random(m)
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.concatenate([r * np.cos(2 * np.pi * u2), r * np.sin(2 * np.pi * u2)])[:n]
    return std * z


def choose_subset(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """Sorted indices of a uniformly random k-subset of range(n)."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    u = g.random(n)
    idx = np.argpartition(u, k - 1)[:k] if k < n else np.arange(n)
    return np.sort(idx.astype(np.int64))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def scale_entries(x: np.ndarray, idx: np.ndarray, factor: float) -> np.ndarray:
    y = x.copy()
    y.reshape(-1)[idx] *= factor
    return y


def scale_columns(x: np.ndarray, cols: np.ndarray, factor: float) -> np.ndarray:
    y = x.copy()
    y[:, cols] *= factor
    return y


# --------------------------------------------------------------------------
# The five workloads.  Shapes are row-major [rows, K] with K contiguous.
# --------------------------------------------------------------------------
CONFIGS = {
    "cfg1": dict(name="mxfp4 quantize->dequantize, fp32 [1,131072], Laplace(0,1) + 1% x50",
                 rows=1, cols=131072),
    "cfg2": dict(name="quantize 4096x4096 bf16 (Gaussian 0.02 | Laplace 0.02 + 16 cols x50)",
                 rows=4096, cols=4096),
    "cfg3": dict(name="fused rotate+quantize 8192x4096 bf16 Laplace(0,1), 8 cols x50",
                 rows=8192, cols=4096),
    "cfg4": dict(name="MXFP4 GEMM M=4096, Llama-3-8B linears",
                 M=4096, KN=[(4096, 4096), (4096, 6144), (4096, 14336), (14336, 4096)]),
    "cfg5": dict(name="Llama-3-70B MLP linears on one GPU",
                 M=[1, 16, 128, 8192], KN=[(8192, 28672), (28672, 8192)]),
}


def cfg1_tensor(seed: int = 0) -> np.ndarray:
    """fp32 [1, 131072]: Laplace(0,1), then 1 % of entries (1311) multiplied by 50."""
    n = 131072
    x = laplace(rng(seed, 1), n, 1.0)
    idx = choose_subset(rng(seed, 101), n, int(round(0.01 * n)))
    return scale_entries(x, idx, 50.0).astype(np.float32).reshape(1, n)


def cfg2_tensor(dist: str, seed: int = 0, rows: int = 4096, cols: int = 4096) -> np.ndarray:
    """bf16 bit patterns [rows, cols].  dist='gauss': N(0, 0.02^2);
    dist='laplace': Laplace(0, 0.02) with 16 random columns (of 4096) x50."""
    if dist == "gauss":
        x = normal(rng(seed, 2), rows * cols, 0.02).reshape(rows, cols)
    elif dist == "laplace":
        x = laplace(rng(seed, 3), rows * cols, 0.02).reshape(rows, cols)
        k = max(1, int(round(16 * cols / 4096)))
        x = scale_columns(x, choose_subset(rng(seed, 103), cols, k), 50.0)
    else:
        raise ValueError(dist)
    return to_bf16_bits(x.astype(np.float32))


def cfg3_tensor(seed: int = 0, rows: int = 8192, cols: int = 4096) -> np.ndarray:
    """bf16 bit patterns [rows, cols]: Laplace(0,1) with 8 of 4096 channels x50."""
    x = laplace(rng(seed, 4), rows * cols, 1.0).reshape(rows, cols)
    k = max(1, int(round(8 * cols / 4096)))
    x = scale_columns(x, choose_subset(rng(seed, 104), cols, k), 50.0)
    return to_bf16_bits(x.astype(np.float32))


def gemm_activation(M: int, K: int, seed: int = 0, outlier_frac: float = 0.002) -> np.ndarray:
    """bf16 bit patterns [M, K]: Laplace(0,1) with round(frac*K) channels x50."""
    x = laplace(rng(seed, 5 + 7 * K), M * K, 1.0).reshape(M, K)
    k = max(1, int(round(outlier_frac * K)))
    x = scale_columns(x, choose_subset(rng(seed, 105 + 7 * K), K, k), 50.0)
    return to_bf16_bits(x.astype(np.float32))


def gemm_weight(N: int, K: int, seed: int = 0, chunk_rows: int = 2048) -> np.ndarray:
    """bf16 bit patterns [N, K] ~ N(0, 0.02^2), generated in row chunks."""
    out = np.empty((N, K), dtype=np.uint16)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        g = rng(seed, 1000003 + 31 * N + 17 * K + r0)
        out[r0:r1] = to_bf16_bits(normal(g, (r1 - r0) * K, 0.02).astype(np.float32)).reshape(r1 - r0, K)
    return out


def random_codes(rows: int, cols: int, seed: int = 0, stream: int = 7) -> np.ndarray:
    """Uniformly random packed 4-bit codes, [rows, cols/2] bytes."""
    return rng(seed, stream).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)


def random_scales(rows: int, nblocks: int, lo: int, hi: int, seed: int = 0,
                  stream: int = 8) -> np.ndarray:
    """Uniformly random scale bytes in [lo, hi], [rows, nblocks]."""
    return rng(seed, stream).integers(lo, hi + 1, size=(rows, nblocks), dtype=np.uint8)


# Kinds of 16-element groups in edge_tensor (one kind per group; an MX block
# holds two groups, an NV block one).
EDGE_KINDS_MX = ("laplace", "tiny", "subnormal", "signed_zeros", "huge", "one_nonzero",
                 "laplace_one_huge")
EDGE_KINDS_NV = ("laplace", "small", "smaller", "subnormal", "signed_zeros", "one_nonzero",
                 "laplace_one_huge")


def edge_tensor(rows: int, cols: int, seed: int = 0, family: str = "mx",
                huge: float = 3.0e38) -> np.ndarray:
    """bf16 bit patterns [rows, cols] whose 16-element groups are each drawn
    from one kind of edge input.  family 'mx' (block scales set by each
    block's own maximum): Laplace(0,1); tiny values 2^-134 .. 2^-126 (block
    maxima below 2^-125, subnormals included); bf16 subnormals only; +0 and
    -0 only; +-huge; a single non-zero element; Laplace with one +-huge
    element.  family 'nv' (one tensor maximum sets the block scales' range):
    Laplace(0,1); Laplace x 1e-5 and x 1e-7 (block maxima far below the tensor
    maximum); bf16 subnormals; signed zeros; a single non-zero; Laplace with
    one element of magnitude `huge`.  Exact bit patterns where the kind needs
    them (subnormals, signed zeros), otherwise fp32 values rounded to bf16."""
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    kinds = EDGE_KINDS_MX if family == "mx" else EDGE_KINDS_NV
    ng = rows * (cols // 16)
    g = rng(seed, 7001)
    kind = g.integers(0, len(kinds), size=ng)
    vals = laplace(rng(seed, 7002), ng * 16, 1.0).reshape(ng, 16)
    sign = np.where(g.random((ng, 16)) < 0.5, -1.0, 1.0)
    pos = g.integers(0, 16, size=ng)
    bits = to_bf16_bits(vals.astype(np.float32)).reshape(ng, 16)
    for k, name in enumerate(kinds):
        m = kind == k
        n = int(m.sum())
        if n == 0 or name == "laplace":
            continue
        if name == "tiny":
            e = g.uniform(-134.0, -126.0, size=(n, 16))
            v = sign[m] * np.exp2(e)
            bits[m] = to_bf16_bits(v.astype(np.float32)).reshape(n, 16)
        elif name == "subnormal":
            mant = g.integers(1, 128, size=(n, 16)).astype(np.uint16)
            bits[m] = np.where(sign[m] < 0, 0x8000, 0).astype(np.uint16) | mant
        elif name == "signed_zeros":
            bits[m] = np.where(sign[m] < 0, 0x8000, 0).astype(np.uint16)
        elif name == "huge":
            v = sign[m] * huge * g.uniform(0.25, 1.0, size=(n, 16))
            bits[m] = to_bf16_bits(v.astype(np.float32)).reshape(n, 16)
        elif name in ("small", "smaller"):
            f = 1e-5 if name == "small" else 1e-7
            bits[m] = to_bf16_bits((vals[m] * f).astype(np.float32)).reshape(n, 16)
        elif name == "one_nonzero":
            row = np.zeros((n, 16), dtype=np.float64)
            row[np.arange(n), pos[m]] = vals[m][np.arange(n), pos[m]] * 7.0
            bits[m] = to_bf16_bits(row.astype(np.float32)).reshape(n, 16)
        elif name == "laplace_one_huge":
            row = vals[m].copy()
            row[np.arange(n), pos[m]] = sign[m][np.arange(n), pos[m]] * huge
            bits[m] = to_bf16_bits(row.astype(np.float32)).reshape(n, 16)
    return bits.reshape(rows, cols)


def extreme_scales(rows: int, nblocks: int, side: str, fmt_mx: bool, seed: int = 0,
                   stream: int = 9, big_codes=(253, 254)) -> np.ndarray:
    """Scale bytes [rows, nblocks] at the ends of the scale formats' ranges,
    paired across the two GEMM operands so that every product of scales stays
    finite.  MX (E8M0): even blocks give side 'a' codes 253/254 and side 'b'
    codes 0/1; odd blocks the reverse (big_codes replaces 253/254); every
    fourth block ordinary codes 120..130 on both sides.  NV (E4M3): subnormal codes 0x01..0x07 and zero
    (0x00) on every other block, ordinary codes 0x30..0x7E elsewhere."""
    g = rng(seed, stream)
    kb = np.arange(nblocks)[None, :]
    if fmt_mx:
        big = g.integers(big_codes[0], big_codes[1] + 1, size=(rows, nblocks))
        small = g.integers(0, 2, size=(rows, nblocks))
        mid = g.integers(120, 131, size=(rows, nblocks))
        a_big = (kb % 2 == 0)
        out = np.where(a_big == (side == "a"), big, small)
        out = np.where(kb % 4 == 3, mid, out)
    else:
        sub = g.integers(0, 8, size=(rows, nblocks))
        mid = g.integers(0x30, 0x7F, size=(rows, nblocks))
        out = np.where(kb % 2 == 0, sub, mid)
    return out.astype(np.uint8)

"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
from __future__ import annotations

import sys

import numpy as np

import fp4_microscaling_quantization_amd as fp4

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def to_dev_u8(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev())


def codes_np(q: fp4.Quantized) -> np.ndarray:
    return fp4.codes_view(q).cpu().numpy()


def rowmajor_scales_np(q: fp4.Quantized) -> np.ndarray:
    """Scales of q gathered into row-major order through fp4_scale_offset."""
    raw = q.scales.cpu().numpy()
    G = q.cfg.block
    nb = q.cols // G
    if q.cfg.scale_layout == fp4.SCALES_ROWMAJOR or q.cfg.fmt not in fp4.MX_FORMATS:
        return raw[: q.rows * nb].reshape(q.rows, nb)
    idx = gemm_offsets(q.rows, q.cols)
    return raw[idx]


_off_cache = {}


def gemm_offsets(rows: int, cols: int) -> np.ndarray:
    """[rows, cols/32] byte offsets of the MXFP4 GEMM scale layout, from the
    library's host-side fp4_scale_offset (sampled, then checked to be the
    affine-in-tiles map it promises to be, then expanded)."""
    key = (rows, cols)
    if key in _off_cache:
        return _off_cache[key]
    cfg = fp4.qconfig(fp4.FMT_MXFP4, scale_layout=fp4.SCALES_GEMM)
    nb = cols // 32
    # offsets of one full tile (32 rows x 8 blocks) plus the tile strides
    r = np.arange(rows)[:, None]
    kb = np.arange(nb)[None, :]
    tile_r = np.minimum(32, rows)
    tile_k = np.minimum(8, nb)
    base = np.array([[fp4.fp4_scale_offset(cfg, rows, cols, i, j) for j in range(tile_k)]
                     for i in range(tile_r)])
    kchunks = (cols + 255) // 256
    off = (r // 32) * kchunks * 256 + (kb // 8) * 256 + base[r % 32, kb % 8]
    # spot-check the expansion against the library at random points
    g = np.random.default_rng(0)
    for _ in range(200):
        i, j = int(g.integers(rows)), int(g.integers(nb))
        assert off[i, j] == fp4.fp4_scale_offset(cfg, rows, cols, i, j)
    _off_cache[key] = off
    return off


def signed_values(codes: np.ndarray) -> np.ndarray:
    c = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def grid_index(vals: np.ndarray) -> np.ndarray:
    """Position on the signed grid -6 .. 6 (15 points; +-0 share index 7)."""
    full = np.concatenate([-GRID[:0:-1], GRID])
    return np.searchsorted(full, vals)


def assert_rotated_codes_close(got_codes, ref_codes, got_scales, ref_scales, budget=1e-4,
                               what=""):
    """Rotated paths: element codes may differ in at most `budget` of the
    elements, and only between adjacent grid points; scale codes in at most
    `budget` of the blocks, by one step."""
    n = got_codes.size * 2
    gv = signed_values(got_codes)
    rv = signed_values(ref_codes)
    diff = gv != rv
    rate = diff.sum() / n
    say("  %s element mismatches: %d of %d (%.2e)" % (what, diff.sum(), n, rate))
    assert rate <= budget, (what, rate)
    if diff.any():
        # compare in the scale of each side's block
        step = np.abs(grid_index(gv[diff]) - grid_index(rv[diff]))
        scale_same = np.repeat(got_scales == ref_scales, gv.shape[1] // got_scales.shape[1], axis=1)[diff]
        assert np.all(step[scale_same] <= 1), (what, "non-adjacent mismatch")
    sd = got_scales != ref_scales
    srate = sd.sum() / got_scales.size
    say("  %s scale mismatches: %d of %d (%.2e)" % (what, sd.sum(), got_scales.size, srate))
    assert srate <= budget, (what, srate)
    if sd.any():
        assert np.all(np.abs(got_scales[sd].astype(int) - ref_scales[sd].astype(int)) == 1)


def gemm_tolerance_ok(got: np.ndarray, ref: np.ndarray, absref: np.ndarray, bf16: bool) -> np.ndarray:
    """|y - y_ref| <= 1e-5 (|A||B|) for fp32 output; for bf16 output the same
    plus half a bf16 ulp of the reference."""
    err = np.abs(got - ref)
    if not bf16:
        return err <= 1e-5 * absref
    return err <= 1e-5 * absref * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)


def assert_search_close(got_codes, got_scales, ref_codes, ref_scales, fmt, ts, y_ref,
                        block_budget=1e-3, elem_budget=1e-4, what=""):
    """Rotated paths under a searching scale rule: the GPU's butterfly sums may
    differ from the oracle's exact ones by an ulp, which can flip a near-tie
    between two candidate scales.  At most `block_budget` of the blocks may
    take another scale, and each such block's squared error (against the
    oracle's rotated values, dequantized by the oracle) must be within 1e-4 of
    the oracle's choice; where the scales agree, element codes follow the
    rotated budget (adjacent points only)."""
    import oracle
    G = fp4.BLOCK[fmt]
    sd = got_scales != ref_scales
    srate = sd.mean()
    say("  %s scale choices differing: %d of %d (%.2e)" % (what, sd.sum(), sd.size, srate))
    assert srate <= block_budget, (what, srate)
    if sd.any():
        yg = oracle.dequantize(got_codes, got_scales, fmt, ts).astype(np.float64)
        yr = oracle.dequantize(ref_codes, ref_scales, fmt, ts).astype(np.float64)
        y = y_ref.astype(np.float64)
        eg = ((yg - y) ** 2).reshape(y.shape[0], -1, G).sum(-1)[sd]
        er = ((yr - y) ** 2).reshape(y.shape[0], -1, G).sum(-1)[sd]
        assert np.all(eg <= er * (1 + 1e-4) + 1e-300), (what, eg[:4], er[:4])
    same = np.repeat(~sd, G // 2, axis=1)
    gv = signed_values(got_codes)
    rv = signed_values(ref_codes)
    diff = (gv != rv) & np.repeat(same, 2, axis=1)
    rate = diff.sum() / gv.size
    say("  %s element mismatches in same-scale blocks: %d (%.2e)" % (what, diff.sum(), rate))
    assert rate <= elem_budget, (what, rate)
    if diff.any():
        assert np.all(np.abs(grid_index(gv[diff]) - grid_index(rv[diff])) <= 1), what


def int4_values(codes: np.ndarray) -> np.ndarray:
    """[rows, cols] integer values of packed two's-complement nibbles."""
    c = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1).astype(np.int64)
    return np.where(c >= 8, c - 16, c)


def assert_rotated_int4_close(got_codes, ref_codes, got_scales, ref_scales, budget=1e-4, what=""):
    """Rotated INT4 paths: element values may differ in at most `budget` of
    the elements, by one integer step, where the block scales agree; scale
    codes in at most `budget` of the blocks, by one step."""
    gv, rv = int4_values(got_codes), int4_values(ref_codes)
    G = gv.shape[1] // got_scales.shape[1]
    same = np.repeat(got_scales == ref_scales, G, axis=1)
    diff = gv != rv
    rate = diff.sum() / gv.size
    say("  %s element mismatches: %d of %d (%.2e)" % (what, diff.sum(), gv.size, rate))
    assert rate <= budget, (what, rate)
    assert np.all(np.abs(gv - rv)[diff & same] <= 1), (what, "non-adjacent mismatch")
    sd = got_scales != ref_scales
    say("  %s scale mismatches: %d of %d" % (what, sd.sum(), sd.size))
    assert sd.mean() <= budget, what
    if sd.any():
        assert np.all(np.abs(got_scales[sd].astype(int) - ref_scales[sd].astype(int)) == 1)

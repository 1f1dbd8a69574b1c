"""Comparison helpers for the GPU parity tests (HIP path vs the oracle).

The tolerance for the normalising ops in reference mode: the per-row
normaliser within 1e-5 relative; dequantised outputs equal except on at most
0.1% of the elements, each of those within one element ulp at the larger of
the two block scales (a block scale can legitimately flip at a power-of-two
boundary when the fp32 and fp64 normalisers differ in the last bits).
"""

import math

import numpy as np
import torch

import oracle

NORM_RTOL = 1e-5
MAX_DIFF_FRACTION = 1e-3


def table(elem):
    return oracle.decode_table(elem)


def unpack_e2m1(packed):
    packed = np.asarray(packed)
    return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[0], -1)


def unpacked(codes, elem):
    return unpack_e2m1(codes) if elem == "e2m1" else np.asarray(codes)


def ulp(u, elem):
    """Spacing of the element grid at |u| (u in element units)."""
    a = np.abs(u)
    emin, mbits = (-6, 3) if elem == "e4m3" else (0, 1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, emin), emin)
    return np.ldexp(1.0, (e - mbits).astype(np.int64))


def compare_reference(codes_g, scales_g, codes_r, scales_r, elem, what=""):
    """Tolerance check against mode (R). Returns the number of differing elements.

    Elements whose block scale and code both agree decode to the same value, so
    only the others are decoded and compared (the outcome is the same as
    decoding every element)."""
    cg, cr = unpacked(codes_g, elem), unpacked(codes_r, elem)
    sg, sr = np.asarray(scales_g), np.asarray(scales_r)
    assert cg.shape == cr.shape and sg.shape == sr.shape
    nan_g, nan_r = sg == 255, sr == 255
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN blocks differ"
    cand = (cg != cr) | np.repeat(sg != sr, 32, axis=1)
    cand &= ~np.repeat(nan_g, 32, axis=1)
    rows, cols = np.nonzero(cand)
    n = 0
    if rows.size:
        tab = table(elem)
        s_g = sg[rows, cols // 32].astype(np.int64)
        s_r = sr[rows, cols // 32].astype(np.int64)
        smax = np.maximum(s_g, s_r)
        ug = tab[cg[rows, cols]] * np.ldexp(1.0, s_g - smax)
        ur = tab[cr[rows, cols]] * np.ldexp(1.0, s_r - smax)
        diff = ug != ur
        n = int(diff.sum())
        if n:
            d = np.abs(ug[diff] - ur[diff])
            lim = ulp(np.maximum(np.abs(ug[diff]), np.abs(ur[diff])), elem)
            worst = float((d / lim).max())
            assert worst <= 1.0, f"{what}: {n} elements differ, worst {worst} ulp"
    # at most 0.1% of the elements, read as ceil(0.001 * N): a tensor of a few
    # hundred elements may show one rounding flip
    assert n <= math.ceil(MAX_DIFF_FRACTION * cg.size), f"{what}: {n} of {cg.size} elements differ"
    return n


FLT_MAX = float(np.finfo(np.float32).max)


def check_normaliser(inv_g, inv_r, what=""):
    """The kernel's fp32 normaliser against the fp64 one: NaN and zero rows
    alike; +Inf exactly where 1/G lies past the fp32 range (up to the
    tolerance); elsewhere within NORM_RTOL relative."""
    inv_g = np.asarray(inv_g, np.float64)
    inv_r = np.asarray(inv_r, np.float64)
    assert np.array_equal(np.isnan(inv_g), np.isnan(inv_r)), f"{what}: NaN rows differ"
    ok = ~np.isnan(inv_r)
    assert np.array_equal(inv_g[ok] == 0, inv_r[ok] == 0), f"{what}: zero rows differ"
    big = ok & np.isposinf(inv_g)
    assert (inv_r[big] * (1 + NORM_RTOL) > FLT_MAX).all(), f"{what}: +Inf normaliser in range"
    nz = ok & (inv_r != 0) & ~big
    if nz.any():
        rel = np.abs(inv_g[nz] - inv_r[nz]) / np.abs(inv_r[nz])
        assert rel.max() <= NORM_RTOL, f"{what}: normaliser off by {rel.max():.3g} relative"


def assert_bf16_bits(a, b, what=""):
    """bf16 bit patterns equal, except that every NaN pattern counts as one
    value (a NaN in the normalised tensor has no defined sign or payload)."""
    a, b = np.asarray(a, np.uint16), np.asarray(b, np.uint16)
    assert a.shape == b.shape, what
    nan_a = (a & 0x7F80) == 0x7F80
    nan_a &= (a & 0x007F) != 0
    nan_b = (b & 0x7F80) == 0x7F80
    nan_b &= (b & 0x007F) != 0
    assert np.array_equal(nan_a, nan_b), f"{what}: NaN positions differ"
    bad = np.argwhere((a != b) & ~nan_a)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}: " \
                          f"{a[tuple(bad[0])]:#06x} vs {b[tuple(bad[0])]:#06x}"


def assert_bits(a, b, what=""):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, what
    bad = np.argwhere(a != b)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}: " \
                          f"{a[tuple(bad[0])]} vs {b[tuple(bad[0])]}"


def host(t):
    return None if t is None else t.detach().cpu()


def np_(t):
    return t.detach().cpu().numpy()

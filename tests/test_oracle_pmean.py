"""Pins of the oracle's MXNorm statistic.

"MXNorm: Reusing MXFP block scales for efficient tensor normalisation"
(gist.science technical summary), §2.1: m_k is the absmax of block k and the
statistic is the power mean G_K^(p) = ((1/K) sum_k m_k^p)^(1/p); §2.2 Theorem 1:
with B fixed and i.i.d. scale-family elements, G converges almost surely to
c(p, B) * RMS; §3.1: p = 1 is the arithmetic mean and p = 2 the quadratic mean.
"""

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.integrate
import scipy.special
import scipy.stats
import torch

from norm_mx_quantisation_amd import workloads


@pytest.mark.parametrize("p", [0.5, 1.0, 2.0, 3.5, 7.0])
def test_pmean_matches_scipy(orc, p):
    rng = np.random.default_rng(31)
    for K in (1, 2, 3, 8, 128, 448):
        m = np.abs(rng.standard_normal(K)) * 10.0 ** rng.uniform(-3, 3)
        got = orc.pmean(m, p)
        want = scipy.stats.pmean(m, p)
        assert got == pytest.approx(want, rel=1e-13)


def test_pmean_special_cases(orc):
    rng = np.random.default_rng(32)
    m = np.abs(rng.standard_normal(128))
    assert orc.pmean(m, 1.0) == pytest.approx(np.mean(m), rel=1e-14)
    assert orc.pmean(m, math.inf) == np.max(m)
    # p -> infinity approaches the maximum from below
    g = [orc.pmean(m, p) for p in (1, 2, 4, 16, 64, 256)]
    assert all(a <= b * (1 + 1e-15) for a, b in zip(g, g[1:]))  # power-mean inequality
    assert abs(orc.pmean(m, 256) - m.max()) < 0.03 * m.max()
    # bracket: max * K^(-1/p) <= G_p <= max
    for p in (0.5, 1, 2, 3.5):
        G = orc.pmean(m, p)
        assert m.max() * len(m) ** (-1 / p) * (1 - 1e-14) <= G <= m.max() * (1 + 1e-14)
    # constant block maxima give G == a for every p
    for p in (0.5, 1, 2, 3.5, math.inf):
        assert orc.pmean(np.full(64, 0.375), p) == pytest.approx(0.375, rel=1e-15)


def test_pmean_exact_rationals(orc):
    getcontext().prec = 50
    rng = np.random.default_rng(33)
    for K in (1, 2, 3, 4):
        m = np.ldexp(rng.integers(1, 256, K).astype(np.float64), rng.integers(-8, 8, K))
        fr = [Fraction(float(v)) for v in m]
        g1 = sum(fr) / K
        assert orc.pmean(m, 1.0) == pytest.approx(float(g1), rel=1e-15)
        s2 = sum(v * v for v in fr) / K
        g2 = (Decimal(s2.numerator) / Decimal(s2.denominator)).sqrt()
        assert orc.pmean(m, 2.0) == pytest.approx(float(g2), rel=1e-15)


def _planted_rows(rng, T, D, lo=0.25, hi=4.0):
    """Rows whose block maxima are planted values with known magnitudes."""
    K = D // 32
    x = rng.uniform(-1, 1, (T, K, 32))
    peaks = rng.uniform(lo, hi, (T, K))
    pos = rng.integers(0, 32, (T, K))
    x = x * peaks[..., None] * 0.5          # every other element is below half the peak
    np.put_along_axis(x, pos[..., None], (peaks * np.where(rng.random((T, K)) < 0.5, -1, 1))[..., None], 2)
    xb = torch.from_numpy(x.reshape(T, D)).to(torch.bfloat16)
    peaks_b = torch.from_numpy(peaks).to(torch.bfloat16).double().numpy()
    return xb, peaks_b


@pytest.mark.parametrize("p", [1.0, 2.0, 3.5, math.inf])
def test_mxnorm_statistic_uses_contiguous_block_maxima(orc, p):
    # planted maxima sit at random positions of contiguous 32-element blocks; a
    # strided or shifted partition would see different maxima
    rng = np.random.default_rng(34)
    xb, peaks = _planted_rows(rng, 16, 512)
    _, _, inv = orc.mxnorm(xb, None, p)
    want = np.array([scipy.stats.pmean(r, p) if math.isfinite(p) else r.max() for r in peaks])
    assert np.allclose(1.0 / inv, want, rtol=1e-14)


def _c_pB(p, B):
    """c(p, B) for N(0,1) elements: (E[M^p])^(1/p), M = max of B i.i.d. |N(0,1)|."""
    tail = lambda m: p * m ** (p - 1) * (1.0 - scipy.special.erf(m / math.sqrt(2.0)) ** B)
    val, _ = scipy.integrate.quad(tail, 0, 60, limit=200)
    return val ** (1.0 / p)


@pytest.mark.parametrize("p", [1.0, 2.0])
def test_theorem1_constant(orc, p):
    # G / RMS over N(0,1) rows concentrates at c(p, 32) (Theorem 1)
    c = _c_pB(p, 32)
    assert 2.3 < c < 2.5
    T, D = 3000, 4096
    x = workloads.random_rows(T, D, seed=35)
    _, _, inv = orc.mxnorm(x, None, p, threads=8)
    xd = x.double().numpy()
    rms = np.sqrt((xd * xd).mean(axis=1))
    ratio = (1.0 / inv) / rms
    sem = ratio.std() / np.sqrt(T)
    assert abs(ratio.mean() - c) < 5 * sem + 1e-3, (ratio.mean(), c, sem)


def test_constant_magnitude_rows_match_rmsnorm(orc):
    # |x_i| = a for all i: every block absmax is a, so G = a = RMS exactly and
    # MXNorm's normaliser equals RMSNorm's with eps = 0
    rng = np.random.default_rng(36)
    for a in (0.375, 3.0, 1.0 / 64):
        x = np.where(rng.random((4, 256)) < 0.5, -a, a)
        xb = torch.from_numpy(x).to(torch.bfloat16)
        for p in (1.0, 2.0, math.inf):
            _, _, inv = orc.mxnorm(xb, None, p)
            assert np.all(inv == 1.0 / a)
        _, _, inv = orc.mxnorm(xb, None, 3.5)   # pow() rounding only
        assert np.allclose(inv, 1.0 / a, rtol=1e-15)
        _, _, _, inv_r = orc.rmsnorm_mxcast(xb, None, eps=0.0)
        assert np.allclose(inv_r, 1.0 / a, rtol=1e-15)

"""Pins of the oracle's straight-through backward.

Reading (MXNorm page, §2.3, gradient paragraph): the backward reuses RMSNorm's
gradient as a straight-through estimator. The cast counts as the identity, and
the forward's exported normaliser inv = 1/G stands where RMSNorm has 1/rms:
    dx_i = inv * g_i - inv^3 * (sum_j g_j x_j / D) * x_i,   g = gamma * dy
    dgamma_i = sum_t dy_ti * x_ti * inv_t.
The pins tie this to torch autograd of RMSNorm. Given RMSNorm's own
normaliser 1/sqrt(mean(x^2) + eps), the formula must be RMSNorm's exact
gradient, which catches a dropped term, a wrong power or sign, or a transposed
reduction. They also check the injected fp32 order against torch's fp32
arithmetic, and MXNorm's normaliser where it equals the RMS one.
"""

import numpy as np
import pytest
import torch

from norm_mx_quantisation_amd import workloads


def bits_to_f64(u16):
    return torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).double().numpy()


def bf16_bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rms_inv(x, eps):
    xd = x.double()
    return (1.0 / torch.sqrt((xd * xd).mean(1) + eps)).float()


def autograd_rmsnorm(x, g, dy, eps):
    xd = x.double().clone().requires_grad_(True)
    gd = g.double().clone().requires_grad_(True)
    y = torch.nn.functional.rms_norm(xd, (x.shape[1],), weight=gd, eps=eps)
    y.backward(dy.double())
    return xd.grad, gd.grad


@pytest.mark.parametrize("D", [32, 256, 4096])
def test_backward_is_rmsnorm_gradient_given_the_rms_normaliser(orc, D):
    eps = 1e-5
    x = workloads.random_rows(12, D, seed=201 + D)
    g = workloads.random_gamma(D, seed=202)
    dy = workloads.random_rows(12, D, seed=203 + D)
    # the normaliser handed to the backward: RMSNorm's own, rounded to fp32,
    # so autograd sees the same value (eps chosen so fp32 inv is its fp64
    # value to 1e-8: the comparison below is on bf16 outputs)
    inv = rms_inv(x, eps)
    dx, s = orc.mxnorm_bwd(x, g, dy, inv.numpy())
    gx, gg = autograd_rmsnorm(x, g, dy, eps)
    want = gx.numpy()
    got = bits_to_f64(dx)
    # dx rounded once to bf16; autograd in fp64 with the exact normaliser
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(want), 1e-30))).astype(np.int64) - 7)
    scale = np.abs(x.double().numpy()) * np.abs(s)[:, None] * inv.double().numpy()[:, None] ** 3 / D
    assert (np.abs(got - want) <= ulp + 1e-6 * (np.abs(want) + scale)).all()
    dgam, absum = orc.mxnorm_bwd_dgamma(x, dy, inv.numpy())
    # inv rounded to fp32 moves each term by at most 2^-24 relative
    assert (np.abs(dgam - gg.numpy()) <= 2.0**-23 * absum + 1e-15).all()


def test_backward_row_dot_and_terms(orc):
    # s is sum_j gamma_j dy_j x_j, each term exact; check against numpy fp64
    x = workloads.random_rows(5, 512, seed=204)
    g = workloads.random_gamma(512, seed=205)
    dy = workloads.random_rows(5, 512, seed=206)
    inv = np.full(5, 0.75, np.float32)
    _, s = orc.mxnorm_bwd(x, g, dy, inv)
    want = (g.double()[None, :] * dy.double() * x.double()).sum(1).numpy()
    assert np.allclose(s, want, rtol=1e-14, atol=0)


def test_backward_gamma_none_is_gamma_ones(orc):
    x = workloads.random_rows(6, 256, seed=207)
    dy = workloads.random_rows(6, 256, seed=208)
    inv = rms_inv(x, 0.0).numpy()
    a = orc.mxnorm_bwd(x, None, dy, inv)
    b = orc.mxnorm_bwd(x, torch.ones(256, dtype=torch.bfloat16), dy, inv)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_backward_injected_mode_follows_fp32_order(orc):
    x = workloads.random_rows(16, 1024, seed=209)
    g = workloads.random_gamma(1024, seed=210)
    dy = workloads.random_rows(16, 1024, seed=211)
    inv = (rms_inv(x, 1e-5) * 2.3).numpy()          # an MXNorm-like normaliser
    _, s64 = orc.mxnorm_bwd(x, g, dy, inv)
    s32 = (s64 * (1 + 2e-7)).astype(np.float32)       # a perturbed fp32 row dot
    dx, s_used = orc.mxnorm_bwd(x, g, dy, inv, s_inject=s32)
    assert (s_used == s32.astype(np.float64)).all()
    a = torch.from_numpy(inv)[:, None]
    k = (a * a) * a
    c = k * (torch.from_numpy(s32)[:, None] / 1024.0)
    gf = g.float()[None, :] * dy.float()
    want = (a * gf - c * x.float()).to(torch.bfloat16)
    assert np.array_equal(dx, bf16_bits(want))


def test_backward_scale_invariance_direction(orc):
    # with RMSNorm's normaliser and eps = 0, the output is invariant to scaling
    # x, so the gradient is orthogonal to x: sum_i x_i dx_i = 0 (before bf16)
    x = workloads.random_rows(4, 2048, seed=212)
    g = workloads.random_gamma(2048, seed=213)
    dy = workloads.random_rows(4, 2048, seed=214)
    inv = rms_inv(x, 0.0).numpy()
    _, s = orc.mxnorm_bwd(x, g, dy, inv)
    xd = x.double().numpy()
    a = inv.astype(np.float64)[:, None]
    gdy = g.double().numpy()[None, :] * dy.double().numpy()
    dx64 = a * gdy - a ** 3 * (s[:, None] / 2048) * xd
    # (x . dx) = inv * s * (1 - inv^2 mean(x^2)), small for the fp32-rounded inv
    dot = (xd * dx64).sum(1)
    ref = np.abs(xd * a * gdy).sum(1)
    assert (np.abs(dot) <= 1e-6 * ref).all()


def test_backward_constant_rows_mxnorm_equals_rmsnorm(orc):
    # |x_i| = a: G = RMS for every p, so MXNorm's normaliser gives RMSNorm's
    # gradient exactly (eps = 0)
    rng = np.random.default_rng(215)
    x = torch.from_numpy(np.where(rng.random((3, 128)) < 0.5, -0.5, 0.5)).to(torch.bfloat16)
    g = workloads.random_gamma(128, seed=216)
    dy = workloads.random_rows(3, 128, seed=217)
    _, _, inv_mx = orc.mxnorm(x, g, 2.0)
    inv_rms = rms_inv(x, 0.0).numpy()
    assert np.array_equal(inv_mx.astype(np.float32), inv_rms)
    a = orc.mxnorm_bwd(x, g, dy, inv_mx.astype(np.float32))
    gx, _ = autograd_rmsnorm(x, g, dy, 0.0)
    assert np.array_equal(a[0], bf16_bits(gx))

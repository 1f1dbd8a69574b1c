"""Tensors past 2^32 elements: [2^20 + 3, 4096] bf16 rows (8 GiB of input).

Element indices, input byte offsets and E4M3 code byte offsets pass 2^32 here
(and on [2^18 + 3, 16384], rows of the split-row and LDS-staged kernels),
and so does the stochastic-rounding counter, which is the element's index
row * D + d (the Philox counter of the SR reading takes all 64 bits of it).
A slip to 32-bit arithmetic anywhere in a kernel's row offsets or in its
counter would show in the last rows. Windows of rows at the start, across
element 2^31 and from just before element 2^32 to the last row are compared
with the oracle, which takes each window's first row, so that its row indices
and counters are the tensor's own. The backward's dgamma, a sum over all rows,
is compared on a few columns over every row. The MX GEMM takes A and C past 4 GiB.
"""

import numpy as np
import pytest
import torch

import norm_mx_quantisation_amd as mxq
import oracle
from norm_mx_quantisation_amd import workloads
from parity_util import assert_bits, host, np_
from test_gpu_nvfp4 import assert_same, check_norm
from test_gpu_parity import (OFFSET, SEED, THREADS, U24, check_mxcast, check_mxnorm,
                             check_rms_fused, check_two_pass, gemm_bound, random_mx_operand)

pytestmark = pytest.mark.gpu
DEV = "cuda"
T, D = (1 << 20) + 3, 4096
WINDOWS = [(0, 16), ((1 << 19) - 8, (1 << 19) + 8), ((1 << 20) - 8, T)]
# rows past 8192: the split-row kernel (and the LDS-staged one, forced)
TW, DW = (1 << 18) + 3, 16384
WIDE_WINDOWS = [(0, 4), ((1 << 17) - 2, (1 << 17) + 2), ((1 << 18) - 2, TW)]


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mxq.lib()
    oracle.lib()
    assert T * D > 1 << 32 and 2 * T * D > 1 << 33
    x = workloads.random_rows(T, D, seed=9001, device=DEV)
    g = workloads.random_gamma(D, seed=9002, device=DEV)
    x[(1 << 20) + 1, :64] *= 100.0   # an outlier block in the last rows
    torch.cuda.synchronize()
    yield x, g
    del x, g
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def wide():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert TW * DW > 1 << 32
    x = workloads.random_rows(TW, DW, seed=9011, device=DEV)
    g = workloads.random_gamma(DW, seed=9012, device=DEV)
    torch.cuda.synchronize()
    yield x, g
    del x, g
    torch.cuda.empty_cache()


def test_mxnorm_sr_past_2_32_elements(big):
    x, g = big
    out = mxq.mxnorm(x, g, 2.0, "e4m3", "sr", SEED, OFFSET)
    torch.cuda.synchronize()
    for w in WINDOWS:
        check_mxnorm(x, g, 2.0, "e4m3", "sr", rows=w, out=out, what=f"mxnorm sr rows {w}")


def test_mxnorm_e2m1_past_2_32_elements(big):
    x, g = big
    out = mxq.mxnorm(x, g, 1.0, "e2m1", "rne", SEED, OFFSET)
    torch.cuda.synchronize()
    for w in WINDOWS:
        check_mxnorm(x, g, 1.0, "e2m1", "rne", rows=w, out=out, what=f"mxnorm e2m1 rows {w}")


def test_mxcast_sr_past_2_32_elements(big):
    x, _ = big
    out = mxq.mxcast(x, "e4m3", "sr", SEED, OFFSET)
    torch.cuda.synchronize()
    for w in WINDOWS:
        check_mxcast(x, "e4m3", "sr", rows=w, out=out, what=f"mxcast sr rows {w}")


def test_two_pass_and_fused_rms_past_2_32_elements(big):
    x, g = big
    w = WINDOWS[-1]
    check_two_pass(x, g, rows=w, what=f"two-pass rows {w}")
    torch.cuda.empty_cache()
    check_rms_fused(x, g, rnd="sr", rows=w, what=f"fused rms sr rows {w}")


def test_nvfp4_past_2_32_elements(big):
    x, g = big
    out = mxq.mxnorm_nvfp4(x, g, 2.0, 1.0)
    torch.cuda.synchronize()
    for r0, r1 in WINDOWS:
        check_norm(x[r0:r1], g, 2.0, 1.0, what=f"mxnorm nvfp4 rows {(r0, r1)}",
                   out=tuple(t[r0:r1] for t in out))
    del out
    c, sc = mxq.nvfp4_cast(x, 1.0)
    torch.cuda.synchronize()
    for r0, r1 in WINDOWS:
        oc, os_ = oracle.nvfp4_cast(host(x[r0:r1]), 1.0, threads=THREADS)
        assert_same(np_(sc[r0:r1]), os_, f"nvfp4 cast scales rows {(r0, r1)}")
        assert_same(np_(c[r0:r1]), oc, f"nvfp4 cast codes rows {(r0, r1)}")


@pytest.mark.parametrize("flags", [0, mxq.MXQ_FLAG_FORCE_LDS])
def test_wide_rows_sr_past_2_32_elements(wide, flags):
    x, g = wide
    out = mxq.mxnorm(x, g, 2.0, "e4m3", "sr", SEED, OFFSET, flags)
    torch.cuda.synchronize()
    for w in WIDE_WINDOWS:
        check_mxnorm(x, g, 2.0, "e4m3", "sr", rows=w, out=out,
                     what=f"wide mxnorm sr flags={flags} rows {w}")


def test_backward_past_2_32_elements(big):
    x, g = big
    _, _, inv = mxq.mxnorm(x, g, 2.0)
    dy = workloads.random_rows(T, D, seed=9003, device=DEV)
    dx, row_dot, dg = mxq.mxnorm_backward(x, g, dy, inv, want_dgamma=True)
    torch.cuda.synchronize()
    gs = host(g)
    for r0, r1 in WINDOWS:
        xs, dys, iv = host(x[r0:r1]), host(dy[r0:r1]), np_(inv[r0:r1])
        ox, _ = oracle.mxnorm_bwd(xs, gs, dys, iv, s_inject=np_(row_dot[r0:r1]), threads=THREADS)
        assert_bits(np_(dx[r0:r1].view(torch.int16)).view(np.uint16), ox,
                    f"bwd dx (I) rows {(r0, r1)}")
    # dgamma on a few columns, each a sum over every row: the partial rows
    # add a slot's rows in order (at most ceil(rows per group / 4)), then 2
    # levels over the slots; the column sum adds up to 16 partial rows per
    # lane in order, a 3-level butterfly and 2 levels over its waves
    cols = torch.tensor([0, 1, 2047, 4095], device=DEV)
    xc, dyc = host(x[:, cols].contiguous()), host(dy[:, cols].contiguous())
    dg64, absum = oracle.mxnorm_bwd_dgamma(xc, dyc, np_(inv))
    rows_per_group = -(-(-(-T // 512)) // 4) * 4   # a multiple of the 4 slots
    n = rows_per_group // 4 + 2 + 16 + 3 + 2 + 2
    got = np_(dg[cols])
    assert (np.abs(got - dg64) <= n * U24 * absum + 1e-30).all(), (got, dg64)
    del dx, row_dot, dg, dy
    torch.cuda.empty_cache()


def test_gemm_past_2_32_bytes():
    """MXFP8 GEMM with A [2^20 + 40, 4096] (4 GiB of codes, a ragged last
    tile) and bf16 C [2^20 + 40, 2048] (4 GiB): rows at the start, across
    byte 2^31 and past byte 2^32 of A and C against the oracle, to the GEMM's
    parity bound."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = (1 << 20) + 40, 2048, 4096
    gen = torch.Generator(device=DEV).manual_seed(9021)
    A = torch.randint(0, 256, (M, K), generator=gen, device=DEV, dtype=torch.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3C                          # no NaN codes
    SA = torch.randint(115, 135, (M, K // 32), generator=gen, device=DEV, dtype=torch.uint8)
    B, SB = random_mx_operand(N, K, seed=9022)
    c = mxq.mx_matmul(A, SA, B, SB, torch.bfloat16)
    torch.cuda.synchronize()
    for r0, r1 in [(0, 8), ((1 << 19) - 4, (1 << 19) + 4), ((1 << 20) - 4, M)]:
        c64, ab = oracle.mx_gemm(np_(A[r0:r1]), np_(SA[r0:r1]), np_(B), np_(SB), K, "e4m3",
                                 "e4m3", threads=THREADS)
        got = c[r0:r1].double().cpu().numpy()
        bound = gemm_bound(ab, K, c64, True)
        assert np.isfinite(c64).all() and np.isfinite(got).all()
        assert (np.abs(got - c64) <= bound).all(), ((r0, r1), np.abs(got - c64).max())
    del A, SA, c
    torch.cuda.empty_cache()

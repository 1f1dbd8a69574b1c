"""Pins of the oracle's MX GEMM: C = A B^T over MX operands.

The MX output of MXNorm feeds the next linear layer, whose gain-folded weight
is MX-cast along K (MXNorm page, §2.3). The pins build expected values test-side
from independent pieces: torch's float8_e4m3fn decode and the golden E2M1
table, the E8M0 scale as 2^(s - 127), and a numpy fp64 matmul of the decoded
matrices. Exact small-integer products check bit equality; per-block scale
edits check that each scale lands on its own rows and 32-column block.
"""

import numpy as np
import pytest
import torch

from test_oracle_formats import _read_table

E2M1 = np.array([v for _, v in _read_table("e2m1_values.txt")])


def e4m3_table():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decode(codes, scales, elem, K):
    if elem == "e2m1":
        lo, hi = codes & 0xF, codes >> 4
        c = np.stack([lo, hi], -1).reshape(codes.shape[0], K)
        v = E2M1[c]
    else:
        v = e4m3_table()[codes]
    s = np.ldexp(1.0, scales.astype(np.int64) - 127).repeat(32, axis=1)
    return v * s


def random_mx(rows, K, elem, rng, lo=118, hi=132):
    if elem == "e2m1":
        codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    else:
        codes = rng.integers(0, 256, (rows, K), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes here
    scales = rng.integers(lo, hi, (rows, K // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("ea,eb", [("e4m3", "e4m3"), ("e2m1", "e2m1"), ("e4m3", "e2m1")])
def test_gemm_matches_decoded_matmul(orc, ea, eb):
    rng = np.random.default_rng(401)
    M, N, K = 9, 13, 256
    A, SA = random_mx(M, K, ea, rng)
    B, SB = random_mx(N, K, eb, rng)
    c, ab = orc.mx_gemm(A, SA, B, SB, K, ea, eb)
    want = decode(A, SA, ea, K) @ decode(B, SB, eb, K).T
    absw = np.abs(decode(A, SA, ea, K)) @ np.abs(decode(B, SB, eb, K)).T
    assert np.allclose(ab, absw, rtol=1e-15, atol=0)
    assert (np.abs(c - want) <= 1e-15 * absw).all()


def test_gemm_exact_on_small_integers(orc):
    # codes of {0, +-1, +-2, +-4} at scale 2^0: every partial sum is a small
    # integer, so the result is exact in any order
    rng = np.random.default_rng(402)
    vals = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x48, 0xC8], np.uint8)
    M, N, K = 5, 7, 512
    A = vals[rng.integers(0, len(vals), (M, K))]
    B = vals[rng.integers(0, len(vals), (N, K))]
    S1 = np.full((M, K // 32), 127, np.uint8)
    S2 = np.full((N, K // 32), 127, np.uint8)
    c, _ = orc.mx_gemm(A, S1, B, S2, K)
    tab = e4m3_table()
    want = (tab[A].astype(np.int64) @ tab[B].astype(np.int64).T)
    assert np.array_equal(c, want.astype(np.float64))


def test_gemm_scale_lands_on_its_block(orc):
    rng = np.random.default_rng(403)
    M, N, K = 4, 6, 128
    A, SA = random_mx(M, K, "e4m3", rng)
    B, SB = random_mx(N, K, "e4m3", rng)
    c0, _ = orc.mx_gemm(A, SA, B, SB, K)
    SA2 = SA.copy()
    SA2[2, 1] += 1                                  # row 2, columns 32..63 doubled
    c1, _ = orc.mx_gemm(A, SA2, B, SB, K)
    tab = e4m3_table()
    blk = (tab[A[2, 32:64]] * np.ldexp(1.0, int(SA[2, 1]) - 127)) @ \
          (tab[B[:, 32:64]] * np.ldexp(1.0, SB[:, 1].astype(np.int64)[:, None] - 127)).T
    assert np.allclose(c1[2] - c0[2], blk, rtol=1e-13, atol=1e-300)
    assert np.array_equal(np.delete(c1, 2, 0), np.delete(c0, 2, 0))
    SB2 = SB.copy()
    SB2[4, 3] = 255                                 # a NaN scale poisons column 4
    c2, _ = orc.mx_gemm(A, SA, B, SB2, K)
    assert np.isnan(c2[:, 4]).all() and np.isfinite(np.delete(c2, 4, 1)).all()


def test_gemm_of_mx_cast_approximates_float_matmul(orc):
    # end to end: MX-cast two float matrices with the oracle's own MXCast and
    # multiply; the result is close to the float product (E4M3 relative error
    # 2^-4 per element)
    rng = np.random.default_rng(404)
    M, N, K = 8, 8, 1024
    x = torch.from_numpy(rng.standard_normal((M, K))).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((N, K))).to(torch.bfloat16)
    A, SA = orc.mxcast(x, "e4m3", "rne")
    B, SB = orc.mxcast(w, "e4m3", "rne")
    c, ab = orc.mx_gemm(A, SA, B, SB, K)
    ref = x.double().numpy() @ w.double().numpy().T
    assert (np.abs(c - ref) <= 2 * 2.0**-4 * ab).all()
    assert np.abs(c - ref).mean() < 0.05 * np.abs(ref).mean()

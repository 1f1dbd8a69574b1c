"""Seeded synthetic inputs for the MXNorm / MXCast workloads.

This module only draws random numbers and shapes them into the workloads'
tensors (bf16 activations and gains). It holds none of the method's
arithmetic: no block maxima, no normalisation, no scales, no codes. Both the
HIP path's tests and the oracle's tests read their inputs from here, so both
sides see identical bytes.

The workloads stand in for the Llama-3 activations of the MXNorm paper
("MXNorm: Reusing MXFP block scales for efficient tensor normalisation",
§3 experiments and §3.2 kernel benchmark), which need trained weights and data
that are not available; every tensor here is synthetic.

Recipe conventions:
  * seed = 1000 + workload index (1..5); generation uses torch.Generator on the
    requested device, so a CPU draw and a GPU draw differ, but each is
    deterministic for its device.
  * fp32 draws are rounded to bf16 with torch's round-to-nearest-even cast.
  * outlier counts are round(fraction * count) with a minimum of 1; which
    channels/rows are outliers comes from a seeded permutation.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

SR_SEED = 0x5EED
SR_OFFSET = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    T: int
    D: int
    description: str
    op: str                  # "mxnorm" or "mxcast"
    p_values: tuple = ()     # p values the workload runs (mxnorm only)
    elem: str = "e4m3"
    roundings: tuple = ("rne",)
    gamma: str = "none"      # "ones", "normal", "uniform" or "none"
    with_two_pass: bool = False

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    w.name: w
    for w in (
        Workload(1, "tiny", 64, 256,
                 "x ~ N(0,1) [64, 256]; gamma = 1 (and gamma = NULL); p = 2; E4M3",
                 "mxnorm", (2.0,), "e4m3", ("rne",), "ones"),
        Workload(2, "llama3_8b_preattn", 8192, 4096,
                 "x ~ N(0,1) [8192, 4096] with 0.1% outlier channels x50; "
                 "gamma ~ 1 + 0.1 N(0,1); p = 1 and p = 2; E4M3; two-pass comparison",
                 "mxnorm", (1.0, 2.0), "e4m3", ("rne",), "normal", True),
        Workload(3, "longseq_t3", 65536, 8192,
                 "x = 0.5 * Student-t(nu=3) [65536, 8192]; gamma ~ U(0.5, 1.5); p = 2; E4M3",
                 "mxnorm", (2.0,), "e4m3", ("rne",), "uniform"),
        Workload(4, "swiglu_downproj", 16384, 14336,
                 "x = silu(a) * b, a, b ~ N(0,1) [16384, 14336], one row in 1000 x100; "
                 "MXCast E4M3 with RNE and with stochastic rounding",
                 "mxcast", (), "e4m3", ("rne", "sr"), "none"),
        Workload(5, "mxfp4", 32768, 4096,
                 "x ~ N(0,1) [32768, 4096] with 1% outlier channels x20; "
                 "gamma ~ 1 + 0.1 N(0,1); p = 2; E2M1 packed two per byte",
                 "mxnorm", (2.0,), "e2m1", ("rne",), "normal"),
    )
}

WORKLOAD_BY_INDEX = {w.index: w for w in WORKLOADS.values()}


def _count(fraction: float, n: int) -> int:
    return max(1, int(round(fraction * n)))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _outlier_index(g: torch.Generator, n: int, k: int, device) -> torch.Tensor:
    return torch.randperm(n, generator=g, device=device)[:k]


def make_inputs(name: str, device="cpu", rows: Optional[int] = None):
    """Return (x bf16 [T, D], gamma bf16 [D] or None) for a named workload.

    ``rows`` truncates T (the first ``rows`` rows of the recipe are produced
    with the same per-row statistics; a truncated draw is not a prefix of the
    full draw).
    """
    w = WORKLOADS[name]
    T = w.T if rows is None else int(rows)
    D = w.D
    device = torch.device(device)
    g = _gen(w.seed, device)
    gamma = None

    if w.name == "tiny":
        x = torch.randn(T, D, generator=g, device=device)
        gamma = torch.ones(D, device=device)
    elif w.name in ("llama3_8b_preattn", "mxfp4"):
        frac, mult = (0.001, 50.0) if w.name == "llama3_8b_preattn" else (0.01, 20.0)
        x = torch.randn(T, D, generator=g, device=device)
        ch = _outlier_index(g, D, _count(frac, D), device)
        x[:, ch] *= mult
        gamma = 1.0 + 0.1 * torch.randn(D, generator=g, device=device)
    elif w.name == "longseq_t3":
        x = torch.empty(T, D, device=device)
        step = max(1, (1 << 26) // D)        # bound the fp32 temporaries
        for r0 in range(0, T, step):
            r1 = min(T, r0 + step)
            z = torch.randn(r1 - r0, D, generator=g, device=device)
            chi = torch.randn(3, r1 - r0, D, generator=g, device=device)
            chi = chi.square_().sum(0).div_(3.0).sqrt_()
            x[r0:r1] = 0.5 * z / chi
        gamma = 0.5 + torch.rand(D, generator=g, device=device)
    elif w.name == "swiglu_downproj":
        x = torch.empty(T, D, device=device)
        step = max(1, (1 << 26) // D)
        for r0 in range(0, T, step):
            r1 = min(T, r0 + step)
            a = torch.randn(r1 - r0, D, generator=g, device=device)
            b = torch.randn(r1 - r0, D, generator=g, device=device)
            x[r0:r1] = torch.nn.functional.silu(a) * b
        rws = _outlier_index(g, T, _count(0.001, T), device)
        x[rws, :] *= 100.0
    else:  # pragma: no cover
        raise KeyError(name)

    xb = x.to(torch.bfloat16).contiguous()
    gb = None if gamma is None else gamma.to(torch.bfloat16).contiguous()
    return xb, gb


def random_rows(T: int, D: int, seed: int, device="cpu", scale: float = 1.0,
                ldx: Optional[int] = None):
    """N(0, scale^2) bf16 rows [T, D] (optionally inside a wider [T, ldx]
    buffer, returned as a strided view) for shape-sweep tests."""
    g = _gen(seed, torch.device(device))
    width = D if ldx is None else ldx
    buf = (scale * torch.randn(T, width, generator=g, device=device)).to(torch.bfloat16)
    return buf[:, :D]


def random_gamma(D: int, seed: int, device="cpu"):
    g = _gen(seed, torch.device(device))
    return (1.0 + 0.1 * torch.randn(D, generator=g, device=device)).to(torch.bfloat16)

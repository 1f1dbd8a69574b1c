"""Time every workload's hot-path call through the C ABI on one GPU.

    python -m norm_mx_quantisation_amd.timing [--steps K] [--only NAME[,NAME]]

For each case: inputs resident in HBM, R rotating buffer sets of at least
1 GB in total (so the 256 MB MALL cannot serve a call), W warm-up launches,
then K launches bracketed by HIP events on the launch stream. Prints one line
per case with the mean time per launch and the algorithmic bandwidth (bytes
the operation must move: read x, write codes and scales; the two-pass path
also writes and reads its bf16 intermediate). Run it under
`rocprofv3 --kernel-trace --stats` for per-kernel durations.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import norm_mx_quantisation_amd as mxq
from norm_mx_quantisation_amd import workloads

HBM_PEAK_GBS = 8000.0

# (case, workload, operation, options)
CASES = (
    ("llama3_8b_preattn mxnorm p=2", "llama3_8b_preattn", "mxnorm", {"p": 2.0}),
    ("llama3_8b_preattn mxnorm p=2 split rows", "llama3_8b_preattn", "mxnorm",
     {"p": 2.0, "flags": mxq.MXQ_FLAG_FORCE_SPLIT}),
    # bytes-only reference kernels with the fused call's traffic and layout
    # (libmxq_floor.so): what moving these bytes alone reaches at this size,
    # then with the normaliser's row dependency and the gain staging added
    ("llama3_8b_preattn floor plain", "llama3_8b_preattn", "floor", {"variant": 0}),
    ("llama3_8b_preattn floor nt loads", "llama3_8b_preattn", "floor", {"variant": 1}),
    ("llama3_8b_preattn floor nt stores", "llama3_8b_preattn", "floor", {"variant": 2}),
    ("llama3_8b_preattn floor nt", "llama3_8b_preattn", "floor", {"variant": 3}),
    ("llama3_8b_preattn floor nt row-gated", "llama3_8b_preattn", "floor", {"variant": 7}),
    ("llama3_8b_preattn floor nt row-gated staged", "llama3_8b_preattn", "floor",
     {"variant": 15}),
    # the same call and floor probe at other row counts (D = 4096, N(0, 1) rows
    # with gains): how much of the launch's ramp and drain the size amortises
    ("rows T=2048 mxnorm p=2", "rows", "mxnorm", {"shape": (2048, 4096)}),
    ("rows T=2048 floor nt row-gated staged", "rows", "floor", {"shape": (2048, 4096), "variant": 15}),
    ("rows T=4096 mxnorm p=2", "rows", "mxnorm", {"shape": (4096, 4096)}),
    ("rows T=4096 floor nt row-gated staged", "rows", "floor", {"shape": (4096, 4096), "variant": 15}),
    ("rows T=16384 mxnorm p=2", "rows", "mxnorm", {"shape": (16384, 4096)}),
    ("rows T=16384 floor nt row-gated staged", "rows", "floor", {"shape": (16384, 4096), "variant": 15}),
    ("rows T=32768 mxnorm p=2", "rows", "mxnorm", {"shape": (32768, 4096)}),
    ("rows T=32768 floor nt row-gated staged", "rows", "floor", {"shape": (32768, 4096), "variant": 15}),
    ("rows T=65536 mxnorm p=2", "rows", "mxnorm", {"shape": (65536, 4096)}),
    ("rows T=65536 floor nt row-gated staged", "rows", "floor", {"shape": (65536, 4096), "variant": 15}),
    ("llama3_8b_preattn mxnorm p=1", "llama3_8b_preattn", "mxnorm", {"p": 1.0}),
    ("llama3_8b_preattn mxnorm p=2 gamma folded", "llama3_8b_preattn", "mxnorm",
     {"p": 2.0, "gamma": False}),
    ("llama3_8b_preattn mxnorm p=2 round-up scales", "llama3_8b_preattn", "mxnorm",
     {"p": 2.0, "flags": mxq.MXQ_FLAG_SCALE_CEIL}),
    ("llama3_8b_preattn rms single-pass", "llama3_8b_preattn", "rms_fused", {}),
    ("llama3_8b_preattn two-pass", "llama3_8b_preattn", "two_pass", {}),
    ("longseq_t3 mxnorm split rows", "longseq_t3", "mxnorm", {}),
    ("longseq_t3 mxnorm register rows", "longseq_t3", "mxnorm",
     {"flags": mxq.MXQ_FLAG_FORCE_REG}),
    ("longseq_t3 mxnorm LDS rows", "longseq_t3", "mxnorm", {"flags": mxq.MXQ_FLAG_FORCE_LDS}),
    # rows wider than one wavefront's registers, N(0,1) with gains, 2^28 elements:
    # the automatic (split-row) kernel and the LDS-staged one
    ("wide D=16384 mxnorm split rows", "wide", "mxnorm", {"shape": (16384, 16384)}),
    ("wide D=16384 mxnorm LDS rows", "wide", "mxnorm",
     {"shape": (16384, 16384), "flags": mxq.MXQ_FLAG_FORCE_LDS}),
    ("wide D=32768 mxnorm split rows", "wide", "mxnorm", {"shape": (8192, 32768)}),
    ("wide D=32768 mxnorm LDS rows", "wide", "mxnorm",
     {"shape": (8192, 32768), "flags": mxq.MXQ_FLAG_FORCE_LDS}),
    # rows that end inside their last 512-element chunk (16352 = 31.9 chunks)
    ("wide D=16352 mxnorm split rows", "wide", "mxnorm", {"shape": (16384, 16352)}),
    ("wide D=16352 mxnorm LDS rows", "wide", "mxnorm",
     {"shape": (16384, 16352), "flags": mxq.MXQ_FLAG_FORCE_LDS}),
    ("swiglu_downproj mxcast rne", "swiglu_downproj", "mxcast", {"rnd": mxq.MXQ_RNE}),
    ("swiglu_downproj mxcast sr", "swiglu_downproj", "mxcast", {"rnd": mxq.MXQ_SR}),
    ("swiglu_downproj mxcast rne round-up scales", "swiglu_downproj", "mxcast",
     {"rnd": mxq.MXQ_RNE, "flags": mxq.MXQ_FLAG_SCALE_CEIL}),
    ("mxfp4 mxnorm e2m1", "mxfp4", "mxnorm", {"elem": mxq.MXQ_E2M1}),
    ("mxfp4 mxnorm e2m1 split rows", "mxfp4", "mxnorm",
     {"elem": mxq.MXQ_E2M1, "flags": mxq.MXQ_FLAG_FORCE_SPLIT}),
    # the same rows in NVFP4 (16-element blocks, E4M3 scales, tensor scale 1)
    ("mxfp4 mxnorm nvfp4", "mxfp4", "nvfp4", {}),
    ("mxfp4 nvfp4 cast", "mxfp4", "nvfp4_cast", {}),
    ("llama3_8b_preattn backward dx+dgamma", "llama3_8b_preattn", "backward", {}),
    ("llama3_8b_preattn backward dx only", "llama3_8b_preattn", "backward", {"dgamma": False}),
    ("mxfp4 backward dx+dgamma", "mxfp4", "backward", {}),
    # MXNormLinear: the MX output of llama3_8b_preattn [8192, 4096] times a
    # gain-folded, MX-cast weight: the QKV projection (4096 + 1024 + 1024 rows)
    # and the feed-forward up projection (14336 rows)
    ("llama3_8b_preattn mx_gemm qkv N=6144", "llama3_8b_preattn", "gemm", {"N": 6144}),
    ("llama3_8b_preattn mx_gemm ffn-up N=14336", "llama3_8b_preattn", "gemm", {"N": 14336}),
    # the same projections in MXFP4: E2M1 activations of mxfp4 [32768, 4096]
    # times an E2M1 weight
    ("mxfp4 mx_gemm e2m1 qkv N=6144", "mxfp4", "gemm", {"N": 6144, "elem": mxq.MXQ_E2M1}),
    ("mxfp4 mx_gemm e2m1 ffn-up N=14336", "mxfp4", "gemm", {"N": 14336, "elem": mxq.MXQ_E2M1}),
    # reference points from the vendor library (hipBLASLt through torch._scaled_mm) at
    # the QKV shape: a plain FP8 GEMM with one scale per tensor, and with 32-element
    # E8M0 block scales
    ("library fp8 per-tensor scaled_mm qkv N=6144", "llama3_8b_preattn", "libgemm", {"N": 6144, "mx": False}),
    ("library mxfp8 block-scaled scaled_mm qkv N=6144", "llama3_8b_preattn", "libgemm", {"N": 6144, "mx": True}),
)

PEAK_MXFP8_TFLOPS = 5000.0    # MI355X dense FP8 / MXFP8 matrix peak
PEAK_MXFP4_TFLOPS = 10100.0   # MI355X dense FP4 / MXFP4 matrix peak


def algorithmic_bytes(op, T, D, elem):
    code = D // 2 if elem == mxq.MXQ_E2M1 else D
    if op == "backward":
        # read x and dy, write dx (bf16), read the normaliser; the dgamma
        # partials are workspace traffic and not counted
        return T * (2 * D + 2 * D + 2 * D + 4)
    if op == "two_pass":
        return T * (2 * D + 2 * D + 2 * D + code + D // 32)
    if op in ("nvfp4", "nvfp4_cast"):
        return T * (2 * D + D // 2 + D // 16)   # E2M1 codes, one E4M3 byte per 16
    return T * (2 * D + code + D // 32)


def run_gemm(torch, name, wl, opt, steps, warmup):
    x0, g = workloads.make_inputs(wl, device="cuda")
    M, K = x0.shape
    N = opt["N"]
    elem = opt.get("elem", mxq.MXQ_E4M3)
    fmt = "e2m1" if elem == mxq.MXQ_E2M1 else "e4m3"
    row = K // 2 if elem == mxq.MXQ_E2M1 else K
    A, SA, _ = mxq.mxnorm(x0, None, 2.0, fmt=fmt)
    w = workloads.random_rows(N, K, seed=11, device="cuda", scale=0.02)
    B, SB = mxq.mxcast((w.float() * g.float()[None, :]).to(torch.bfloat16), fmt=fmt)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L = mxq.lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    args = (vp(A.data_ptr()), row, vp(SA.data_ptr()), K // 32, vp(B.data_ptr()), row,
            vp(SB.data_ptr()), K // 32, M, N, K, elem, elem, vp(C.data_ptr()), N, mxq.MXQ_OUT_BF16,
            stream)

    def launch(i):
        st = L.mx_gemm(*args)
        if st != mxq.MXQ_OK:
            raise mxq.MxqError(st, name)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        launch(i)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    peak, pname = ((PEAK_MXFP4_TFLOPS, "MXFP4") if elem == mxq.MXQ_E2M1
                   else (PEAK_MXFP8_TFLOPS, "MXFP8"))
    print(f"{name:44s} M={M:6d} N={N:6d} K={K:5d} {us:9.2f} us/launch (events, back-to-back)  "
          f"{tflops:8.1f} TFLOP/s  {100 * tflops / peak:5.1f}% of {pname} peak",
          flush=True)
    del A, SA, B, SB, C
    torch.cuda.empty_cache()


def run_libgemm(torch, name, wl, opt, steps, warmup):
    w = workloads.WORKLOADS[wl]
    M, K, N = w.T, w.D, opt["N"]
    g = torch.Generator().manual_seed(12)
    a = (torch.randn(M, K, generator=g) * 0.5).to(torch.float8_e4m3fn).to("cuda")
    b = (torch.randn(N, K, generator=g) * 0.5).to(torch.float8_e4m3fn).to("cuda")
    if opt["mx"]:
        sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
        sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
    else:
        sa = sb = torch.tensor(1.0, device="cuda")
    try:
        f = lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
    except (RuntimeError, TypeError) as e:
        print(f"{name:44s} not available in this torch build: {str(e)[:120]}", flush=True)
        return
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        f()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    print(f"{name:44s} M={M:6d} N={N:6d} K={K:5d} {us:9.2f} us/launch (events, back-to-back)  "
          f"{tflops:8.1f} TFLOP/s  {100 * tflops / PEAK_MXFP8_TFLOPS:5.1f}% of MXFP8 peak", flush=True)


_floor = None


def floor_lib():
    """libmxq_floor.so, the bytes-only reference kernels (built with libmxq.so)."""
    global _floor
    if _floor is None:
        path = os.path.join(os.path.dirname(mxq.LIB_PATH), "libmxq_floor.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run norm_mx_quantisation_amd.build")
        L = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.mxq_floor_stream.argtypes = [vp, vp, i64, i64, vp, vp, ctypes.c_int, vp]
        L.mxq_floor_stream.restype = ctypes.c_int
        _floor = L
    return _floor


def run_case(torch, name, wl, op, opt, steps, warmup):
    if op == "gemm":
        return run_gemm(torch, name, wl, opt, steps, warmup)
    if op == "libgemm":
        return run_libgemm(torch, name, wl, opt, steps, warmup)
    if "shape" in opt:
        T, D = opt["shape"]
        x0 = workloads.random_rows(T, D, seed=13, device="cuda")
        g = workloads.random_gamma(D, seed=14, device="cuda")
    else:
        x0, g = workloads.make_inputs(wl, device="cuda")
    T, D = x0.shape
    if not opt.get("gamma", True):
        g = None
    elem = opt.get("elem", mxq.MXQ_E4M3)
    rnd = opt.get("rnd", mxq.MXQ_RNE)
    rng = mxq.mxq_rng(workloads.SR_SEED, workloads.SR_OFFSET)
    x_bytes = x0.numel() * 2
    R = max(2, min(10, -(-(1 << 30) // x_bytes)))      # >= 1 GB of inputs in rotation
    nv = op in ("nvfp4", "nvfp4_cast")
    cb = D // 2 if (elem == mxq.MXQ_E2M1 or nv) else D
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    codes = [torch.empty((T, cb), dtype=torch.uint8, device="cuda") for _ in range(R)]
    scales = [torch.empty((T, D // 16 if nv else D // 32), dtype=torch.uint8, device="cuda")
              for _ in range(R)]
    invs = [torch.empty((T,), dtype=torch.float32, device="cuda") for _ in range(R)]
    ys = ([torch.empty((T, D), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
          if op in ("two_pass", "backward") else None)
    if op == "backward":
        R = max(2, min(10, -(-(1 << 30) // (3 * x_bytes))))
        xs, ys = xs[:R], ys[:R]
        dys = [workloads.random_rows(T, D, seed=7 + k, device="cuda") for k in range(R)]
        for k in range(R):
            mxq.mxnorm(xs[k], g, 2.0, out=(codes[k], scales[k], invs[k]))
        want_dg = opt.get("dgamma", True)
        dgam = torch.empty((D,), dtype=torch.float32, device="cuda")
        wsb = mxq.mxnorm_bwd_workspace_size(T, D)
        ws = torch.empty((wsb // 4,), dtype=torch.float32, device="cuda")
        rows = torch.empty((T,), dtype=torch.float32, device="cuda")
    L = mxq.lib()
    vp = ctypes.c_void_p
    gp = vp(g.data_ptr()) if g is not None else None
    stream = vp(torch.cuda.current_stream().cuda_stream)
    rngp = ctypes.pointer(rng) if rnd == mxq.MXQ_SR else None

    def launch(i):
        k = i % R
        xp, cp, sp, ip = (vp(xs[k].data_ptr()), vp(codes[k].data_ptr()),
                          vp(scales[k].data_ptr()), vp(invs[k].data_ptr()))
        if op == "mxnorm":
            st = L.mxnorm_fwd(xp, D, gp, T, D, ctypes.c_float(opt.get("p", 2.0)), elem, rnd, rngp,
                              opt.get("flags", 0), cp, sp, ip, stream)
        elif op == "rms_fused":
            st = L.rmsnorm_mxcast_fused_fwd(xp, D, gp, T, D, ctypes.c_float(1e-5), elem, rnd, rngp,
                                            0, cp, sp, ip, stream)
        elif op == "backward":
            st = L.mxnorm_bwd(xp, D, gp, vp(dys[k].data_ptr()), D, ip, T, D, vp(ys[k].data_ptr()),
                              vp(rows.data_ptr()), vp(dgam.data_ptr()) if want_dg else None,
                              vp(ws.data_ptr()) if want_dg else None, wsb if want_dg else 0,
                              stream)
        elif op == "two_pass":
            st = L.rmsnorm_mxcast_fwd(xp, D, gp, T, D, ctypes.c_float(1e-5), elem, rnd, rngp,
                                      opt.get("flags", 0), vp(ys[k].data_ptr()), cp, sp, ip,
                                      stream)
        elif op == "nvfp4":
            st = L.mxnorm_nvfp4_fwd(xp, D, gp, T, D, ctypes.c_float(opt.get("p", 2.0)),
                                    ctypes.c_float(1.0), cp, sp, ip, stream)
        elif op == "nvfp4_cast":
            st = L.nvfp4_cast_fwd(xp, D, T, D, ctypes.c_float(1.0), cp, sp, stream)
        elif op == "floor":
            st = floor_lib().mxq_floor_stream(xp, gp, T, D, cp, sp, opt["variant"], stream)
        else:
            st = L.mxcast_fwd(xp, D, T, D, elem, rnd, rngp, opt.get("flags", 0), cp, sp, stream)
        if st != mxq.MXQ_OK:
            raise mxq.MxqError(st, name)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        launch(i)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    nbytes = algorithmic_bytes(op, T, D, elem)
    gbs = nbytes / (us * 1e-6) / 1e9
    print(f"{name:44s} T={T:6d} D={D:6d} {us:9.2f} us/launch (events, back-to-back)  "
          f"{nbytes:>13,d} B  {gbs:8.1f} GB/s  {100 * gbs / HBM_PEAK_GBS:5.1f}% of HBM peak",
          flush=True)
    del xs, codes, scales, invs, ys
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        print("timing needs a GPU", file=sys.stderr)
        sys.exit(1)
    sel = [s for s in args.only.split(",") if s]
    for name, wl, op, opt in CASES:
        if sel and not any(s in name for s in sel):
            continue
        run_case(torch, name, wl, op, opt, args.steps, args.warmup)


if __name__ == "__main__":
    main()

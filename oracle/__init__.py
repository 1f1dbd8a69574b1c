"""Python access to the scalar C oracle (mxq_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path never imports this
package and shares no code with it.

Inputs are numpy arrays (uint16 bf16 bit patterns) or CPU torch bf16 tensors.
Row work is split over Python threads; ctypes releases the GIL inside each
foreign call, so the C loops run in parallel.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

E4M3, E2M1 = 0, 1
RNE, SR = 0, 1
ELEM = {"e4m3": E4M3, "e2m1": E2M1}
RND = {"rne": RNE, "sr": SR}
RULE = {"floor": 0, "ceil": 1}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain IEEE, no contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-shared",
             "-fPIC", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build(force=True)
            L = ctypes.CDLL(LIB)
            i64, u64, i32, u32, dbl = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                                       ctypes.c_uint32, ctypes.c_double)
            vp = ctypes.c_void_p
            L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
            L.orc_bf16_to_f64.restype = dbl
            L.orc_bf16_rne.argtypes = [dbl]
            L.orc_bf16_rne.restype = ctypes.c_uint16
            L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.orc_e4m3_decode.restype = dbl
            L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
            L.orc_e2m1_decode.restype = dbl
            L.orc_encode.argtypes = [i32, i32, dbl, u32]
            L.orc_encode.restype = ctypes.c_uint8
            L.orc_encode_array.argtypes = [i32, i32, vp, vp, i64, vp]
            L.orc_encode_array.restype = None
            L.orc_e8m0_scale.argtypes = [i32, dbl]
            L.orc_e8m0_scale.restype = ctypes.c_uint8
            L.orc_e8m0_scale_rule.argtypes = [i32, dbl, i32]
            L.orc_e8m0_scale_rule.restype = ctypes.c_uint8
            L.orc_philox4x32_10.argtypes = [vp, vp, vp]
            L.orc_philox4x32_10.restype = None
            L.orc_philox4x64_10.argtypes = [vp, vp, vp]
            L.orc_philox4x64_10.restype = None
            L.orc_sr_word.argtypes = [u64, u64, u64]
            L.orc_sr_word.restype = u32
            L.orc_sr_words.argtypes = [u64, u64, u64, i64, vp]
            L.orc_sr_words.restype = None
            L.orc_pmean.argtypes = [vp, i64, dbl]
            L.orc_pmean.restype = dbl
            L.orc_mxcast_f64.argtypes = [vp, i64, i64, i32, i32, i32, u64, u64, vp, vp]
            L.orc_mxcast_f64.restype = i32
            L.orc_mxcast.argtypes = [vp, i64, i64, i64, i32, i32, i32, u64, u64, i64, vp, vp]
            L.orc_mxcast.restype = i32
            L.orc_mxnorm.argtypes = [vp, i64, vp, i64, i64, dbl, i32, i32, i32, u64, u64, i64,
                                     vp, vp, vp, vp]
            L.orc_mxnorm.restype = i32
            L.orc_rmsnorm_mxcast.argtypes = [vp, i64, vp, i64, i64, dbl, i32, i32, i32, u64, u64,
                                             i64, vp, vp, vp, vp, vp]
            L.orc_rmsnorm_mxcast.restype = i32
            L.orc_rmsnorm_fused_mxcast.argtypes = [vp, i64, vp, i64, i64, dbl, i32, i32, i32, u64,
                                                   u64, i64, vp, vp, vp, vp]
            L.orc_rmsnorm_fused_mxcast.restype = i32
            L.orc_mxnorm_bwd.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, vp, vp, vp]
            L.orc_mxnorm_bwd.restype = i32
            L.orc_mxnorm_bwd_dgamma.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp, vp]
            L.orc_mxnorm_bwd_dgamma.restype = i32
            L.orc_mx_gemm.argtypes = [vp, i64, vp, i64, i32, vp, i64, vp, i64, i32, i64, i64,
                                      i64, vp, vp]
            L.orc_mx_gemm.restype = i32
            L.orc_nvfp4_cast.argtypes = [vp, i64, i64, i64, dbl, vp, vp]
            L.orc_nvfp4_cast.restype = i32
            L.orc_mxnorm_nvfp4.argtypes = [vp, i64, vp, i64, i64, dbl, dbl, vp, vp, vp, vp]
            L.orc_mxnorm_nvfp4.restype = i32
            L.orc_nvfp4_block.argtypes = [vp, dbl, i32, vp, vp]
            L.orc_nvfp4_block.restype = i32
            _lib = L
    return _lib


# --------------------------------------------------------------------------
# input marshalling
# --------------------------------------------------------------------------

def as_bf16_bits(x) -> np.ndarray:
    """uint16 view of a bf16 tensor / uint16 array (2-D, unit column stride)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            assert x.dtype == torch.bfloat16 and x.device.type == "cpu"
            return x.view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    assert a.dtype == np.uint16
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _rows_view(x: np.ndarray):
    if x.ndim == 1:
        x = x.reshape(1, -1)
    assert x.ndim == 2 and x.strides[1] == 2, "columns must be contiguous"
    T, D = x.shape
    ldx = x.strides[0] // 2 if T > 1 else D
    return x, T, D, ldx


def _split(T: int, threads: int):
    threads = max(1, min(threads, T)) if T else 1
    step = (T + threads - 1) // threads if T else 0
    return [(r0, min(T, r0 + step)) for r0 in range(0, T, step)] if T else []


def _run(jobs, threads):
    if threads <= 1 or len(jobs) <= 1:
        rcs = [j() for j in jobs]
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            rcs = list(ex.map(lambda j: j(), jobs))
    for rc in rcs:
        if rc != 0:
            raise ValueError(f"oracle returned error {rc}")


def code_bytes(elem: int, D: int) -> int:
    return D // 2 if elem == E2M1 else D


# --------------------------------------------------------------------------
# the operations
# --------------------------------------------------------------------------

def mxcast(x, elem="e4m3", rnd="rne", seed=0, offset=0, row_base=0, threads=1, rule="floor"):
    """MXCast (R mode is the only mode: the result is unique). Returns (codes, scales)."""
    L = lib()
    e, r, ru = ELEM[elem], RND[rnd], RULE[rule]
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    codes = np.zeros((T, code_bytes(e, D)), np.uint8)
    scales = np.zeros((T, D // 32), np.uint8)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_mxcast(ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, r1 - r0, D, e, r,
                                    ru, seed, offset, row_base + r0, _ptr(codes[r0:]),
                                    _ptr(scales[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return codes, scales


def mxnorm(x, gamma=None, p=2.0, elem="e4m3", rnd="rne", seed=0, offset=0,
           inv_inject=None, row_base=0, threads=1, rule="floor"):
    """Fused MXNorm -> MX cast. inv_inject=None: mode (R); else mode (I) with the
    given fp32 per-row normalisers. Returns (codes, scales, inv float64 [T])."""
    L = lib()
    e, r = ELEM[elem], RND[rnd]
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    g = None if gamma is None else np.ascontiguousarray(as_bf16_bits(gamma).reshape(-1))
    inj = None if inv_inject is None else np.ascontiguousarray(
        np.asarray(inv_inject, dtype=np.float32).reshape(-1))
    codes = np.zeros((T, code_bytes(e, D)), np.uint8)
    scales = np.zeros((T, D // 32), np.uint8)
    inv = np.zeros(T, np.float64)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_mxnorm(
            ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, _ptr(g), r1 - r0, D, float(p), e, r,
            RULE[rule], seed, offset, row_base + r0, None if inj is None else _ptr(inj[r0:]),
            _ptr(codes[r0:]), _ptr(scales[r0:]), _ptr(inv[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return codes, scales, inv


def nvfp4_cast(x, tensor_scale=1.0, threads=1):
    """NVFP4 cast of bf16 rows: (codes [T, D/2] packed E2M1, scales [T, D/16] E4M3)."""
    L = lib()
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    codes = np.zeros((T, D // 2), np.uint8)
    scales = np.zeros((T, D // 16), np.uint8)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_nvfp4_cast(ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, r1 - r0, D,
                                        float(tensor_scale), _ptr(codes[r0:]), _ptr(scales[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return codes, scales


def mxnorm_nvfp4(x, gamma=None, p=2.0, tensor_scale=1.0, inv_inject=None, threads=1):
    """MXNorm over NVFP4 blocks. inv_inject=None: mode (R); else mode (I) with the
    given fp32 per-row normalisers. Returns (codes, scales, inv float64 [T])."""
    L = lib()
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    g = None if gamma is None else np.ascontiguousarray(as_bf16_bits(gamma).reshape(-1))
    inj = None if inv_inject is None else np.ascontiguousarray(
        np.asarray(inv_inject, dtype=np.float32).reshape(-1))
    codes = np.zeros((T, D // 2), np.uint8)
    scales = np.zeros((T, D // 16), np.uint8)
    inv = np.zeros(T, np.float64)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_mxnorm_nvfp4(
            ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, _ptr(g), r1 - r0, D, float(p),
            float(tensor_scale), None if inj is None else _ptr(inj[r0:]), _ptr(codes[r0:]),
            _ptr(scales[r0:]), _ptr(inv[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return codes, scales, inv


def nvfp4_block(v, tensor_scale=1.0, fp32=True):
    """NVFP4 encode of one block of 16 values: (16 unpacked E2M1 codes, E4M3 scale byte)."""
    L = lib()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(16))
    codes = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    rc = L.orc_nvfp4_block(_ptr(a), float(tensor_scale), int(bool(fp32)), _ptr(codes), _ptr(sc))
    if rc != 0:
        raise ValueError(f"oracle returned error {rc}")
    return codes, int(sc[0])


def rmsnorm_mxcast(x, gamma=None, eps=1e-5, elem="e4m3", rnd="rne", seed=0, offset=0,
                   inv_inject=None, row_base=0, threads=1, rule="floor"):
    """Two-pass RMSNorm (bf16 y) -> MXCast(y). Returns (y uint16, codes, scales, inv)."""
    L = lib()
    e, r = ELEM[elem], RND[rnd]
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    g = None if gamma is None else np.ascontiguousarray(as_bf16_bits(gamma).reshape(-1))
    inj = None if inv_inject is None else np.ascontiguousarray(
        np.asarray(inv_inject, dtype=np.float32).reshape(-1))
    y = np.zeros((T, D), np.uint16)
    codes = np.zeros((T, code_bytes(e, D)), np.uint8)
    scales = np.zeros((T, D // 32), np.uint8)
    inv = np.zeros(T, np.float64)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_rmsnorm_mxcast(
            ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, _ptr(g), r1 - r0, D, float(eps), e, r,
            RULE[rule], seed, offset, row_base + r0, None if inj is None else _ptr(inj[r0:]),
            _ptr(y[r0:]), _ptr(codes[r0:]), _ptr(scales[r0:]), _ptr(inv[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return y, codes, scales, inv


def rmsnorm_fused_mxcast(x, gamma=None, eps=1e-5, elem="e4m3", rnd="rne", seed=0, offset=0,
                         inv_inject=None, row_base=0, threads=1, rule="floor"):
    """Single-pass exact-RMS normalise and MX cast (y not rounded to bf16).
    Returns (codes, scales, inv float64 [T])."""
    L = lib()
    e, r = ELEM[elem], RND[rnd]
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    g = None if gamma is None else np.ascontiguousarray(as_bf16_bits(gamma).reshape(-1))
    inj = None if inv_inject is None else np.ascontiguousarray(
        np.asarray(inv_inject, dtype=np.float32).reshape(-1))
    codes = np.zeros((T, code_bytes(e, D)), np.uint8)
    scales = np.zeros((T, D // 32), np.uint8)
    inv = np.zeros(T, np.float64)
    xb = x.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_rmsnorm_fused_mxcast(
            ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, _ptr(g), r1 - r0, D, float(eps), e, r,
            RULE[rule], seed, offset, row_base + r0, None if inj is None else _ptr(inj[r0:]),
            _ptr(codes[r0:]), _ptr(scales[r0:]), _ptr(inv[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return codes, scales, inv


def mxnorm_bwd(x, gamma, dy, inv, s_inject=None, threads=1):
    """Straight-through backward: returns (dx uint16 bf16 bits [T, D], s float64 [T]).
    s_inject=None: mode (R); else mode (I) with the given fp32 row dots."""
    L = lib()
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    d, T2, D2, lddy = _rows_view(as_bf16_bits(dy))
    assert (T2, D2) == (T, D)
    g = None if gamma is None else np.ascontiguousarray(as_bf16_bits(gamma).reshape(-1))
    iv = np.ascontiguousarray(np.asarray(inv, dtype=np.float32).reshape(-1))
    inj = None if s_inject is None else np.ascontiguousarray(
        np.asarray(s_inject, dtype=np.float32).reshape(-1))
    dx = np.zeros((T, D), np.uint16)
    s = np.zeros(T, np.float64)
    xb, db = x.ctypes.data, d.ctypes.data

    def job(r0, r1):
        return lambda: L.orc_mxnorm_bwd(
            ctypes.c_void_p(xb + 2 * r0 * ldx), ldx, _ptr(g), ctypes.c_void_p(db + 2 * r0 * lddy),
            lddy, _ptr(iv[r0:]), r1 - r0, D, None if inj is None else _ptr(inj[r0:]),
            _ptr(dx[r0:]), _ptr(s[r0:]))
    _run([job(a, b) for a, b in _split(T, threads)], threads)
    return dx, s


def mxnorm_bwd_dgamma(x, dy, inv):
    """dgamma [D] float64 and the matching sum of |terms| per column."""
    L = lib()
    x, T, D, ldx = _rows_view(as_bf16_bits(x))
    d, _, _, lddy = _rows_view(as_bf16_bits(dy))
    iv = np.ascontiguousarray(np.asarray(inv, dtype=np.float32).reshape(-1))
    out = np.zeros(D, np.float64)
    ab = np.zeros(D, np.float64)
    rc = L.orc_mxnorm_bwd_dgamma(_ptr(x), ldx, _ptr(d), lddy, _ptr(iv), T, D, _ptr(out), _ptr(ab))
    if rc:
        raise ValueError(f"oracle returned error {rc}")
    return out, ab


def mx_gemm(a_codes, a_scales, b_codes, b_scales, K, elem_a="e4m3", elem_b="e4m3",
            threads=1):
    """C = A B^T over MX operands (codes [rows, K or K/2] uint8, scales [rows, K/32]).
    Returns (C float64 [M, N], sum |a b| float64 [M, N])."""
    L = lib()
    A = np.ascontiguousarray(np.asarray(a_codes, dtype=np.uint8))
    SA = np.ascontiguousarray(np.asarray(a_scales, dtype=np.uint8))
    B = np.ascontiguousarray(np.asarray(b_codes, dtype=np.uint8))
    SB = np.ascontiguousarray(np.asarray(b_scales, dtype=np.uint8))
    M, N = A.shape[0], B.shape[0]
    c = np.zeros((M, N), np.float64)
    ab = np.zeros((M, N), np.float64)
    ea, eb = ELEM[elem_a], ELEM[elem_b]

    def job(r0, r1):
        return lambda: L.orc_mx_gemm(
            ctypes.c_void_p(A.ctypes.data + r0 * A.shape[1]), A.shape[1],
            ctypes.c_void_p(SA.ctypes.data + r0 * SA.shape[1]), SA.shape[1], ea,
            _ptr(B), B.shape[1], _ptr(SB), SB.shape[1], eb, r1 - r0, N, K,
            _ptr(c[r0:]), _ptr(ab[r0:]))
    _run([job(x, y) for x, y in _split(M, threads)], threads)
    return c, ab


# --------------------------------------------------------------------------
# element-level helpers (for the pins)
# --------------------------------------------------------------------------

def decode(elem, c: int) -> float:
    L = lib()
    return L.orc_e2m1_decode(c) if ELEM.get(elem, elem) == E2M1 else L.orc_e4m3_decode(c)


def encode(elem, rnd, v: float, r: int = 0) -> int:
    return lib().orc_encode(ELEM.get(elem, elem), RND.get(rnd, rnd), float(v), int(r))


def encode_array(elem, rnd, v, r=None) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
    rr = None if r is None else np.ascontiguousarray(np.asarray(r, dtype=np.uint32).reshape(-1))
    out = np.zeros(a.size, np.uint8)
    lib().orc_encode_array(ELEM.get(elem, elem), RND.get(rnd, rnd), _ptr(a), _ptr(rr), a.size,
                           _ptr(out))
    return out


def e8m0_scale(elem, amax: float, rule="floor") -> int:
    if rule == "floor":
        return lib().orc_e8m0_scale(ELEM.get(elem, elem), float(amax))
    return lib().orc_e8m0_scale_rule(ELEM.get(elem, elem), float(amax), RULE[rule])


def pmean(m, p: float) -> float:
    a = np.ascontiguousarray(np.asarray(m, dtype=np.float64))
    return lib().orc_pmean(_ptr(a), a.size, float(p))


def bf16_rne(v: float) -> int:
    return lib().orc_bf16_rne(float(v))


def philox4x32(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox4x64(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    out = np.zeros(4, np.uint64)
    lib().orc_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed: int, offset: int, n: int) -> int:
    return lib().orc_sr_word(seed, offset, n)


def sr_words(seed: int, offset: int, n0: int, count: int) -> np.ndarray:
    out = np.zeros(count, np.uint32)
    lib().orc_sr_words(seed, offset, n0, count, _ptr(out))
    return out


def mxcast_f64(v, elem="e4m3", rnd="rne", seed=0, offset=0, t=0, rule="floor"):
    """MXCast of one row of doubles; returns (unpacked codes [D], scales [D/32])."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
    D = a.size
    codes = np.zeros(D, np.uint8)
    scales = np.zeros(D // 32, np.uint8)
    rc = lib().orc_mxcast_f64(_ptr(a), D, t, ELEM[elem], RND[rnd], RULE[rule], seed, offset,
                              _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError(f"oracle returned error {rc}")
    return codes, scales


def decode_table(elem) -> np.ndarray:
    e = ELEM.get(elem, elem)
    n = 16 if e == E2M1 else 256
    return np.array([decode(e, c) for c in range(n)], dtype=np.float64)

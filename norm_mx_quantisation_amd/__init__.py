"""norm_mx_quantisation_amd: MXNorm fused with the MX cast on MI355X (gfx950).

Thin ctypes binding of libmxq.so. The functions named like the C entry points
(mxnorm_fwd, rmsnorm_mxcast_fwd, rmsnorm_mxcast_fused_fwd, mxcast_fwd,
mxnorm_bwd, mxnorm_bwd_noalloc, mx_gemm, nvfp4_cast_fwd, mxnorm_nvfp4_fwd,
mxq_strerror, mxq_abi_version) take raw device pointers and sizes and return
the status code, exactly as the C ABI does. The torch helpers (mxnorm,
rmsnorm_mxcast, rmsnorm_mxcast_fused, mxcast, mxnorm_backward, mx_matmul,
nvfp4_cast, mxnorm_nvfp4) only check tensor metadata, allocate the outputs and
pass pointers; every step of the computation runs in the HIP kernels.
mx_views reinterprets outputs as torch's float8/float4 dtypes without a copy.
There is no CPU fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxq.so")

MXQ_OK, MXQ_ERR_NULL, MXQ_ERR_SHAPE, MXQ_ERR_ALIGN, MXQ_ERR_ARG, MXQ_ERR_UNSUPPORTED, MXQ_ERR_HIP = range(7)
MXQ_E4M3, MXQ_E2M1 = 0, 1
MXQ_RNE, MXQ_SR = 0, 1
MXQ_FLAG_FORCE_REG, MXQ_FLAG_FORCE_LDS, MXQ_FLAG_SCALE_CEIL, MXQ_FLAG_FORCE_SPLIT = 1, 2, 4, 8
MXQ_OUT_F32, MXQ_OUT_BF16 = 0, 1
MXQ_MAX_D_REG, MXQ_MAX_D = 8192, 32768
ABI_VERSION = 4

EXPORTS = ("mxnorm_fwd", "rmsnorm_mxcast_fwd", "rmsnorm_mxcast_fused_fwd", "mxcast_fwd",
           "mxnorm_bwd", "mxnorm_bwd_workspace_size", "mxnorm_bwd_noalloc", "mx_gemm",
           "nvfp4_cast_fwd", "mxnorm_nvfp4_fwd", "mxq_strerror", "mxq_abi_version")


class mxq_rng(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


class MxqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({mxq_strerror(status)})")


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded libmxq.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"libmxq.so is not built ({LIB_PATH}); run "
                    "`python -m norm_mx_quantisation_amd.build` or __graft_entry__.build()")
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, f32, i32, u32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_uint32)
            rp = ctypes.POINTER(mxq_rng)
            L.mxnorm_fwd.argtypes = [vp, i64, vp, i64, i64, f32, i32, i32, rp, u32, vp, vp, vp, vp]
            L.mxnorm_fwd.restype = i32
            L.rmsnorm_mxcast_fwd.argtypes = [vp, i64, vp, i64, i64, f32, i32, i32, rp, u32, vp, vp,
                                             vp, vp, vp]
            L.rmsnorm_mxcast_fwd.restype = i32
            L.rmsnorm_mxcast_fused_fwd.argtypes = [vp, i64, vp, i64, i64, f32, i32, i32, rp, u32,
                                                   vp, vp, vp, vp]
            L.rmsnorm_mxcast_fused_fwd.restype = i32
            L.mxcast_fwd.argtypes = [vp, i64, i64, i64, i32, i32, rp, u32, vp, vp, vp]
            L.mxcast_fwd.restype = i32
            L.mxnorm_bwd.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
            L.mxnorm_bwd.restype = i32
            L.mxnorm_bwd_noalloc.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, vp, vp, vp, vp]
            L.mxnorm_bwd_noalloc.restype = i32
            L.mxnorm_bwd_workspace_size.argtypes = [i64, i64]
            L.mxnorm_bwd_workspace_size.restype = ctypes.c_size_t
            L.mx_gemm.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, i32, i32, vp,
                                  i64, i32, vp]
            L.mx_gemm.restype = i32
            L.nvfp4_cast_fwd.argtypes = [vp, i64, i64, i64, f32, vp, vp, vp]
            L.nvfp4_cast_fwd.restype = i32
            L.mxnorm_nvfp4_fwd.argtypes = [vp, i64, vp, i64, i64, f32, f32, vp, vp, vp, vp]
            L.mxnorm_nvfp4_fwd.restype = i32
            L.mxq_strerror.argtypes = [i32]
            L.mxq_strerror.restype = ctypes.c_char_p
            L.mxq_abi_version.argtypes = []
            L.mxq_abi_version.restype = i32
            if L.mxq_abi_version() != ABI_VERSION:
                raise RuntimeError("libmxq.so ABI version mismatch")
            _lib = L
    return _lib


def _rng(rng) -> Optional[ctypes.POINTER(mxq_rng)]:
    if rng is None:
        return None
    if isinstance(rng, mxq_rng):
        return ctypes.pointer(rng)
    seed, offset = rng
    return ctypes.pointer(mxq_rng(seed, offset))


# ---------------------------------------------------------------- raw C entry points

def mxnorm_fwd(x, ldx, gamma, T, D, p, elem, rnd, rng, flags, codes, scales, inv_norm,
               stream) -> int:
    return lib().mxnorm_fwd(x, ldx, gamma, T, D, p, elem, rnd, _rng(rng), flags, codes, scales,
                            inv_norm, stream)


def rmsnorm_mxcast_fwd(x, ldx, gamma, T, D, eps, elem, rnd, rng, flags, y_workspace, codes,
                       scales, inv_rms, stream) -> int:
    return lib().rmsnorm_mxcast_fwd(x, ldx, gamma, T, D, eps, elem, rnd, _rng(rng), flags,
                                    y_workspace, codes, scales, inv_rms, stream)


def rmsnorm_mxcast_fused_fwd(x, ldx, gamma, T, D, eps, elem, rnd, rng, flags, codes, scales,
                             inv_rms, stream) -> int:
    return lib().rmsnorm_mxcast_fused_fwd(x, ldx, gamma, T, D, eps, elem, rnd, _rng(rng), flags,
                                          codes, scales, inv_rms, stream)


def mxcast_fwd(x, ldx, T, D, elem, rnd, rng, flags, codes, scales, stream) -> int:
    return lib().mxcast_fwd(x, ldx, T, D, elem, rnd, _rng(rng), flags, codes, scales, stream)


def nvfp4_cast_fwd(x, ldx, T, D, tensor_scale, codes, scales, stream) -> int:
    return lib().nvfp4_cast_fwd(x, ldx, T, D, tensor_scale, codes, scales, stream)


def mxnorm_nvfp4_fwd(x, ldx, gamma, T, D, p, tensor_scale, codes, scales, inv_norm,
                     stream) -> int:
    return lib().mxnorm_nvfp4_fwd(x, ldx, gamma, T, D, p, tensor_scale, codes, scales, inv_norm,
                                  stream)


def mxnorm_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma, workspace,
               workspace_bytes, stream) -> int:
    return lib().mxnorm_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma,
                            workspace, workspace_bytes, stream)


def mxnorm_bwd_noalloc(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma,
                       stream) -> int:
    return lib().mxnorm_bwd_noalloc(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma,
                                    stream)


def mxnorm_bwd_workspace_size(T, D) -> int:
    return lib().mxnorm_bwd_workspace_size(T, D)


def mx_gemm(a, lda, a_scales, ldsa, b, ldb, b_scales, ldsb, M, N, K, elem_a, elem_b, c, ldc,
            c_type, stream) -> int:
    return lib().mx_gemm(a, lda, a_scales, ldsa, b, ldb, b_scales, ldsb, M, N, K, elem_a, elem_b,
                         c, ldc, c_type, stream)


def mxq_strerror(status: int) -> str:
    return lib().mxq_strerror(status).decode()


def mxq_abi_version() -> int:
    return lib().mxq_abi_version()


# ---------------------------------------------------------------- torch helpers

_ELEM = {"e4m3": MXQ_E4M3, "e2m1": MXQ_E2M1}
_RND = {"rne": MXQ_RNE, "sr": MXQ_SR}
_RULE = {"floor": 0, "ceil": MXQ_FLAG_SCALE_CEIL}   # E8M0 scale rule -> flag bit


def _check_x(x):
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    if not x.is_cuda:
        raise ValueError("x must live on the GPU (there is no CPU path)")
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    T, D = x.shape
    return T, D, (x.stride(0) if T > 1 else D)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_buf(t, what, shape, dtype, device, optional=False):
    """A caller-supplied buffer must match exactly what the kernel writes or
    reads: a contiguous tensor of this dtype and shape on the input's device
    (a wrong size or a host tensor would be an out-of-bounds GPU access)."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError(f"{what} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be {dtype} of shape {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.device != device:
        raise ValueError(f"{what} must live on {device}, got {t.device}")


def _check_gamma(gamma, D, device):
    import torch
    _check_buf(gamma, "gamma", (D,), torch.bfloat16, device, optional=True)


def _check_outputs(out, T, D, elem, device, want_inv):
    """out = (codes, scales[, inv]) from a caller; checked like _outputs' own."""
    import torch
    if not isinstance(out, (tuple, list)) or len(out) not in (2, 3):
        raise ValueError("out must be (codes, scales) or (codes, scales, inv)")
    codes, scales = out[0], out[1]
    inv = out[2] if len(out) == 3 else None
    cb = D // 2 if elem == MXQ_E2M1 else D
    _check_buf(codes, "codes", (T, cb), torch.uint8, device)
    _check_buf(scales, "scales", (T, D // 32), torch.uint8, device)
    if want_inv:
        _check_buf(inv, "inv", (T,), torch.float32, device, optional=True)
    return codes, scales, inv


def _outputs(x, T, D, elem, want_inv):
    import torch
    cb = D // 2 if elem == MXQ_E2M1 else D
    codes = torch.empty((T, cb), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, D // 32), dtype=torch.uint8, device=x.device)
    inv = torch.empty((T,), dtype=torch.float32, device=x.device) if want_inv else None
    return codes, scales, inv


def mxnorm(x, gamma=None, p: float = 2.0, fmt: str = "e4m3", rounding: str = "rne", seed: int = 0,
           offset: int = 0, flags: int = 0, stream=None, out=None, scale_rule: str = "floor"):
    """Fused MXNorm -> MX cast. Returns (codes uint8, scales uint8 E8M0, inv_norm fp32).
    scale_rule "floor" (OCP) or "ceil" (round the E8M0 scale up: no saturation)."""
    T, D, ldx = _check_x(x)
    elem, rnd = _ELEM[fmt], _RND[rounding]
    flags |= _RULE[scale_rule]
    codes, scales, inv = (_check_outputs(out, T, D, elem, x.device, True) if out is not None
                          else _outputs(x, T, D, elem, True))
    _check_gamma(gamma, D, x.device)
    st = mxnorm_fwd(_ptr(x), ldx, _ptr(gamma), T, D, float(p), elem, rnd,
                    (seed, offset) if rnd == MXQ_SR else None, flags, _ptr(codes), _ptr(scales),
                    _ptr(inv), _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "mxnorm_fwd")
    return codes, scales, inv


def rmsnorm_mxcast(x, gamma=None, eps: float = 1e-5, fmt: str = "e4m3", rounding: str = "rne",
                   seed: int = 0, offset: int = 0, stream=None, out=None, y=None,
                   scale_rule: str = "floor"):
    """Two-pass RMSNorm (bf16 y) -> MXCast. Returns (codes, scales, inv_rms, y)."""
    import torch
    T, D, ldx = _check_x(x)
    elem, rnd = _ELEM[fmt], _RND[rounding]
    flags = _RULE[scale_rule]
    codes, scales, inv = (_check_outputs(out, T, D, elem, x.device, True) if out is not None
                          else _outputs(x, T, D, elem, True))
    _check_gamma(gamma, D, x.device)
    if y is None:
        y = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    _check_buf(y, "y", (T, D), torch.bfloat16, x.device)
    st = rmsnorm_mxcast_fwd(_ptr(x), ldx, _ptr(gamma), T, D, float(eps), elem, rnd,
                            (seed, offset) if rnd == MXQ_SR else None, flags, _ptr(y),
                            _ptr(codes), _ptr(scales), _ptr(inv), _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "rmsnorm_mxcast_fwd")
    return codes, scales, inv, y


def rmsnorm_mxcast_fused(x, gamma=None, eps: float = 1e-5, fmt: str = "e4m3",
                         rounding: str = "rne", seed: int = 0, offset: int = 0, flags: int = 0,
                         stream=None, out=None, scale_rule: str = "floor"):
    """Single-pass exact-RMS normalise and MX cast. Returns (codes, scales, inv_rms)."""
    T, D, ldx = _check_x(x)
    elem, rnd = _ELEM[fmt], _RND[rounding]
    flags |= _RULE[scale_rule]
    codes, scales, inv = (_check_outputs(out, T, D, elem, x.device, True) if out is not None
                          else _outputs(x, T, D, elem, True))
    _check_gamma(gamma, D, x.device)
    st = rmsnorm_mxcast_fused_fwd(_ptr(x), ldx, _ptr(gamma), T, D, float(eps), elem, rnd,
                                  (seed, offset) if rnd == MXQ_SR else None, flags, _ptr(codes),
                                  _ptr(scales), _ptr(inv), _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "rmsnorm_mxcast_fused_fwd")
    return codes, scales, inv


def mxcast(x, fmt: str = "e4m3", rounding: str = "rne", seed: int = 0, offset: int = 0,
           stream=None, out=None, scale_rule: str = "floor"):
    """MXCast. Returns (codes, scales)."""
    T, D, ldx = _check_x(x)
    elem, rnd = _ELEM[fmt], _RND[rounding]
    codes, scales, _ = (_check_outputs(out, T, D, elem, x.device, False) if out is not None
                        else _outputs(x, T, D, elem, False))
    st = mxcast_fwd(_ptr(x), ldx, T, D, elem, rnd, (seed, offset) if rnd == MXQ_SR else None,
                    _RULE[scale_rule], _ptr(codes), _ptr(scales), _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "mxcast_fwd")
    return codes, scales


def mx_views(codes, scales, fmt: str = "e4m3"):
    """torch dtype views of the uint8 outputs, no copy: E4M3 codes as float8_e4m3fn, packed
    E2M1 codes as float4_e2m1fn_x2 (two elements per byte, element 2j in the low nibble), E8M0
    scales as float8_e8m0fnu, NVFP4's E4M3 scales (fmt "nvfp4") as float8_e4m3fn."""
    import torch
    if fmt not in ("e4m3", "e2m1", "nvfp4"):
        raise ValueError('fmt must be "e4m3", "e2m1" or "nvfp4"')
    cv = codes.view(torch.float8_e4m3fn) if fmt == "e4m3" else codes.view(torch.float4_e2m1fn_x2)
    sv = scales.view(torch.float8_e4m3fn) if fmt == "nvfp4" else scales.view(torch.float8_e8m0fnu)
    return cv, sv


def _nvfp4_outputs(x, T, D, out, want_inv):
    import torch
    if out is None:
        codes = torch.empty((T, D // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((T, D // 16), dtype=torch.uint8, device=x.device)
        inv = torch.empty((T,), dtype=torch.float32, device=x.device) if want_inv else None
        return codes, scales, inv
    if not isinstance(out, (tuple, list)) or len(out) not in (2, 3):
        raise ValueError("out must be (codes, scales) or (codes, scales, inv)")
    codes, scales = out[0], out[1]
    inv = out[2] if len(out) == 3 else None
    _check_buf(codes, "codes", (T, D // 2), torch.uint8, x.device)
    _check_buf(scales, "scales", (T, D // 16), torch.uint8, x.device)
    if want_inv:
        _check_buf(inv, "inv", (T,), torch.float32, x.device, optional=True)
    return codes, scales, inv


def nvfp4_cast(x, tensor_scale: float = 1.0, stream=None, out=None):
    """NVFP4 cast. Returns (codes uint8 [T, D/2] packed E2M1, scales uint8 [T, D/16] E4M3)."""
    T, D, ldx = _check_x(x)
    codes, scales, _ = _nvfp4_outputs(x, T, D, out, False)
    st = nvfp4_cast_fwd(_ptr(x), ldx, T, D, tensor_scale, _ptr(codes), _ptr(scales),
                        _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "nvfp4_cast_fwd")
    return codes, scales


def mxnorm_nvfp4(x, gamma=None, p: float = 2.0, tensor_scale: float = 1.0, stream=None,
                 out=None):
    """MXNorm over NVFP4 blocks. Returns (codes, scales E4M3 [T, D/16], inv_norm fp32)."""
    T, D, ldx = _check_x(x)
    _check_gamma(gamma, D, x.device)
    codes, scales, inv = _nvfp4_outputs(x, T, D, out, True)
    st = mxnorm_nvfp4_fwd(_ptr(x), ldx, _ptr(gamma), T, D, p, tensor_scale, _ptr(codes),
                          _ptr(scales), _ptr(inv), _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "mxnorm_nvfp4_fwd")
    return codes, scales, inv


def mxnorm_backward(x, gamma, dy, inv_norm, want_dgamma: bool = True, stream=None, out=None):
    """Straight-through backward. Returns (dx bf16, row_dot fp32, dgamma fp32 or None).
    out = (dx, row_dot, dgamma, workspace) reuses caller buffers."""
    import torch
    T, D, ldx = _check_x(x)
    Td, Dd, lddy = _check_x(dy)
    if (Td, Dd) != (T, D):
        raise ValueError("dy must have the shape of x")
    if dy.device != x.device:
        raise ValueError("dy must live on the device of x")
    if (not isinstance(inv_norm, torch.Tensor) or inv_norm.dtype != torch.float32
            or inv_norm.numel() != T or not inv_norm.is_contiguous() or inv_norm.device != x.device):
        raise ValueError("inv_norm must be a contiguous fp32 tensor of T elements on x's device")
    _check_gamma(gamma, D, x.device)
    if out is not None:
        dx, row_dot, dgamma, ws = out
        _check_buf(dx, "dx", (T, D), torch.bfloat16, x.device)
        _check_buf(row_dot, "row_dot", (T,), torch.float32, x.device)
        _check_buf(dgamma, "dgamma", (D,), torch.float32, x.device, optional=True)
        if dgamma is not None:
            if ws is None:
                raise ValueError("dgamma needs a workspace")
            _check_buf(ws, "workspace", tuple(ws.shape), ws.dtype, x.device)
    else:
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
        row_dot = torch.empty((T,), dtype=torch.float32, device=x.device)
        dgamma = torch.empty((D,), dtype=torch.float32, device=x.device) if want_dgamma else None
        nb = mxnorm_bwd_workspace_size(T, D) if want_dgamma else 0
        ws = torch.empty((max(nb, 16) // 4,), dtype=torch.float32, device=x.device) if want_dgamma else None
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = mxnorm_bwd(_ptr(x), ldx, _ptr(gamma), _ptr(dy), lddy, _ptr(inv_norm), T, D, _ptr(dx),
                    _ptr(row_dot), _ptr(dgamma), _ptr(ws), nbytes, _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "mxnorm_bwd")
    return dx, row_dot, dgamma


def mx_matmul(a_codes, a_scales, b_codes, b_scales, out_dtype=None, stream=None, out=None,
              fmt_a: str = "e4m3", fmt_b: str = "e4m3"):
    """C = A B^T for MX operands: uint8 codes [M, K] / [N, K] (E4M3) or [M, K/2] /
    [N, K/2] (packed E2M1, per fmt_a / fmt_b), E8M0 scales [M, K/32] / [N, K/32].
    out_dtype torch.float32 (default) or torch.bfloat16."""
    import torch
    for t in (a_codes, a_scales, b_codes, b_scales):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 2 or not t.is_cuda:
            raise TypeError("MX operands must be 2-D uint8 GPU tensors")
        if t.stride(1) != 1:
            raise ValueError("MX operands need unit column stride")
    if fmt_a not in _ELEM or fmt_b not in _ELEM:
        raise ValueError(f"fmt_a / fmt_b must be one of {sorted(_ELEM)}")
    ea, eb = _ELEM[fmt_a], _ELEM[fmt_b]
    per_byte = lambda e: 2 if e == MXQ_E2M1 else 1   # elements per code byte
    M = a_codes.shape[0]
    N = b_codes.shape[0]
    K = a_codes.shape[1] * per_byte(ea)
    if (b_codes.shape[1] * per_byte(eb) != K or a_scales.shape != (M, K // 32)
            or b_scales.shape != (N, K // 32)):
        raise ValueError("MX operand shapes do not match")
    dev = a_codes.device
    if any(t.device != dev for t in (a_scales, b_codes, b_scales)):
        raise ValueError("MX operands must live on one device")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    ct = {torch.float32: MXQ_OUT_F32, torch.bfloat16: MXQ_OUT_BF16}[out_dtype]
    if out is not None:
        # the kernel writes M rows of N elements of out_dtype at out's row stride
        if not isinstance(out, torch.Tensor) or out.dtype != out_dtype or tuple(out.shape) != (M, N):
            raise ValueError(f"out must be {out_dtype} of shape {(M, N)}")
        if out.device != dev or (N > 1 and out.stride(1) != 1) or (M > 1 and out.stride(0) < N):
            raise ValueError("out must be on the operands' device with unit column stride")
    c = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    ld = lambda t: t.stride(0) if t.shape[0] > 1 else t.shape[1]
    st = mx_gemm(_ptr(a_codes), ld(a_codes), _ptr(a_scales), ld(a_scales), _ptr(b_codes),
                 ld(b_codes), _ptr(b_scales), ld(b_scales), M, N, K, ea, eb, _ptr(c),
                 ld(c) if M > 1 else N, ct, _stream(stream))
    if st != MXQ_OK:
        raise MxqError(st, "mx_gemm")
    return c


def as_torch_mx(codes, scales, fmt: str = "e4m3"):
    """Views of the outputs as torch's float8_e4m3fn / float4_e2m1fn_x2 and float8_e8m0fnu."""
    import torch
    c = codes.view(torch.float8_e4m3fn) if fmt == "e4m3" else codes.view(torch.float4_e2m1fn_x2)
    return c, scales.view(torch.float8_e8m0fnu)

"""C-ABI checks that need no GPU: the library loads, exports every function
include/mxq.h declares, and rejects bad arguments before any HIP call.

Every call here fails validation, so no kernel is ever launched (fake device
pointers are never dereferenced).
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

import norm_mx_quantisation_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")

A16 = 0x10000       # a 16-byte aligned fake device address (never dereferenced)
A8 = A16 + 8        # 8-byte aligned, not 16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(mxq.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.check_output(["nm", "-D", "--defined-only", mxq.LIB_PATH], text=True)
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for fn in declared_functions():
        assert fn in names, fn
        assert hasattr(mxq.lib(), fn)


def test_abi_version_and_messages():
    assert mxq.mxq_abi_version() == mxq.ABI_VERSION == 4
    for st in range(7):
        assert isinstance(mxq.mxq_strerror(st), str) and mxq.mxq_strerror(st)
    assert mxq.mxq_strerror(99) == "unknown status"


def norm(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, T=8, D=4096, p=2.0, elem=0, rnd=0, rng=None, flags=0,
             codes=A16, scales=A16, inv_norm=None, stream=None)
    a.update(kw)
    return mxq.mxnorm_fwd(a["x"], a["ldx"], a["gamma"], a["T"], a["D"], a["p"], a["elem"], a["rnd"],
                          a["rng"], a["flags"], a["codes"], a["scales"], a["inv_norm"], a["stream"])


def rms(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, T=8, D=4096, eps=1e-5, elem=0, rnd=0, rng=None,
             flags=0, y=A16, codes=A16, scales=A16, inv=None, stream=None)
    a.update(kw)
    return mxq.rmsnorm_mxcast_fwd(a["x"], a["ldx"], a["gamma"], a["T"], a["D"], a["eps"], a["elem"],
                                  a["rnd"], a["rng"], a["flags"], a["y"], a["codes"], a["scales"],
                                  a["inv"], a["stream"])


def rms_fused(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, T=8, D=4096, eps=1e-5, elem=0, rnd=0, rng=None,
             flags=0, codes=A16, scales=A16, inv=None, stream=None)
    a.update(kw)
    return mxq.rmsnorm_mxcast_fused_fwd(a["x"], a["ldx"], a["gamma"], a["T"], a["D"], a["eps"],
                                        a["elem"], a["rnd"], a["rng"], a["flags"], a["codes"],
                                        a["scales"], a["inv"], a["stream"])


def cast(**kw):
    a = dict(x=A16, ldx=4096, T=8, D=4096, elem=0, rnd=0, rng=None, flags=0, codes=A16,
             scales=A16, stream=None)
    a.update(kw)
    return mxq.mxcast_fwd(a["x"], a["ldx"], a["T"], a["D"], a["elem"], a["rnd"], a["rng"],
                          a["flags"], a["codes"], a["scales"], a["stream"])


def nvcast(**kw):
    a = dict(x=A16, ldx=4096, T=8, D=4096, ts=1.0, codes=A16, scales=A16, stream=None)
    a.update(kw)
    return mxq.nvfp4_cast_fwd(a["x"], a["ldx"], a["T"], a["D"], a["ts"], a["codes"], a["scales"],
                              a["stream"])


def nvnorm(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, T=8, D=4096, p=2.0, ts=1.0, codes=A16, scales=A16,
             inv=None, stream=None)
    a.update(kw)
    return mxq.mxnorm_nvfp4_fwd(a["x"], a["ldx"], a["gamma"], a["T"], a["D"], a["p"], a["ts"],
                                a["codes"], a["scales"], a["inv"], a["stream"])


@pytest.mark.parametrize("call", [nvcast, nvnorm])
def test_nvfp4_argument_errors(call):
    assert call(D=0) == mxq.MXQ_ERR_SHAPE
    assert call(D=4000 + 16) == mxq.MXQ_ERR_SHAPE
    assert call(T=-1) == mxq.MXQ_ERR_SHAPE
    assert call(ldx=2048) == mxq.MXQ_ERR_SHAPE
    for ts in (0.0, -1.0, float("nan"), float("inf"), 2.0 ** -33, 2.0 ** 33):
        assert call(ts=ts) == mxq.MXQ_ERR_ARG, ts
    assert call(D=8224, ldx=8224) == mxq.MXQ_ERR_UNSUPPORTED   # one wavefront per row: D <= 8192
    assert call(x=None) == mxq.MXQ_ERR_NULL
    assert call(codes=None) == mxq.MXQ_ERR_NULL
    assert call(scales=None) == mxq.MXQ_ERR_NULL
    assert call(x=A8) == mxq.MXQ_ERR_ALIGN
    assert call(codes=A8) == mxq.MXQ_ERR_ALIGN
    assert call(ldx=4100) == mxq.MXQ_ERR_ALIGN
    assert call(T=0, x=None, codes=None, scales=None) == mxq.MXQ_OK    # empty: nothing to do
    assert call(T=1 << 34, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED


def test_mxnorm_nvfp4_argument_errors():
    for p in (0.0, -1.0, float("nan")):
        assert nvnorm(p=p) == mxq.MXQ_ERR_ARG
    assert nvnorm(gamma=A8) == mxq.MXQ_ERR_ALIGN
    assert nvnorm(inv=A16 + 2) == mxq.MXQ_ERR_ALIGN


@pytest.mark.parametrize("call", [norm, rms, rms_fused, cast])
def test_shape_errors(call):
    assert call(D=0) == mxq.MXQ_ERR_SHAPE
    assert call(D=-32) == mxq.MXQ_ERR_SHAPE
    assert call(D=4000 + 16) == mxq.MXQ_ERR_SHAPE       # not a multiple of 32
    assert call(T=-1) == mxq.MXQ_ERR_SHAPE
    assert call(ldx=2048) == mxq.MXQ_ERR_SHAPE          # ldx < D


@pytest.mark.parametrize("call", [norm, rms, rms_fused, cast])
def test_null_and_alignment_errors(call):
    assert call(x=None) == mxq.MXQ_ERR_NULL
    assert call(codes=None) == mxq.MXQ_ERR_NULL
    assert call(scales=None) == mxq.MXQ_ERR_NULL
    assert call(x=A8) == mxq.MXQ_ERR_ALIGN
    assert call(codes=A8) == mxq.MXQ_ERR_ALIGN
    assert call(ldx=4100) == mxq.MXQ_ERR_ALIGN          # rows not 16-byte aligned


@pytest.mark.parametrize("call", [norm, rms, rms_fused, cast])
def test_format_rounding_rng_errors(call):
    assert call(elem=2) == mxq.MXQ_ERR_ARG
    assert call(rnd=5) == mxq.MXQ_ERR_ARG
    assert call(rnd=1, rng=None) == mxq.MXQ_ERR_ARG     # SR needs a stream


def test_sizes_past_the_launch_limits():
    # Refused on the host before any HIP call (the pointers are never used).
    # 32-element rows keep T * D below the 2^40 element limit.
    huge = 1 << 34   # 2^32 workgroups of 4 rows: past the grid limit
    assert norm(T=huge, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED
    assert rms_fused(T=huge, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED
    # 2^32 chunks of 512 elements: past the cast pass's 32-bit chunk count
    assert rms(T=1 << 32, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED
    assert cast(T=1 << 32, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED
    # past the element limit
    assert norm(T=1 << 35, D=32, ldx=32) == mxq.MXQ_ERR_UNSUPPORTED


def test_mxnorm_argument_errors():
    assert norm(p=0.0) == mxq.MXQ_ERR_ARG
    assert norm(p=-1.0) == mxq.MXQ_ERR_ARG
    assert norm(p=float("nan")) == mxq.MXQ_ERR_ARG
    assert norm(flags=3) == mxq.MXQ_ERR_ARG                      # two variants forced
    assert norm(flags=mxq.MXQ_FLAG_FORCE_SPLIT | mxq.MXQ_FLAG_FORCE_LDS) == mxq.MXQ_ERR_ARG
    assert norm(flags=mxq.MXQ_FLAG_FORCE_SPLIT | mxq.MXQ_FLAG_FORCE_REG) == mxq.MXQ_ERR_ARG
    assert norm(flags=16) == mxq.MXQ_ERR_ARG                     # unknown bit
    assert norm(flags=mxq.MXQ_FLAG_SCALE_CEIL | 3) == mxq.MXQ_ERR_ARG
    assert norm(D=8224, ldx=8224, flags=mxq.MXQ_FLAG_FORCE_REG) == mxq.MXQ_ERR_UNSUPPORTED
    assert norm(D=mxq.MXQ_MAX_D + 32, ldx=mxq.MXQ_MAX_D + 32) == mxq.MXQ_ERR_UNSUPPORTED
    assert norm(D=mxq.MXQ_MAX_D + 32, ldx=mxq.MXQ_MAX_D + 32,
                flags=mxq.MXQ_FLAG_FORCE_SPLIT) == mxq.MXQ_ERR_UNSUPPORTED
    assert norm(gamma=A8) == mxq.MXQ_ERR_ALIGN
    assert norm(inv_norm=A16 + 2) == mxq.MXQ_ERR_ALIGN


def test_rms_fused_argument_errors():
    assert rms_fused(eps=-1e-6) == mxq.MXQ_ERR_ARG
    assert rms_fused(eps=float("nan")) == mxq.MXQ_ERR_ARG
    assert rms_fused(eps=float("inf")) == mxq.MXQ_ERR_ARG
    assert rms_fused(flags=3) == mxq.MXQ_ERR_ARG
    assert rms_fused(D=8224, ldx=8224, flags=mxq.MXQ_FLAG_FORCE_REG) == mxq.MXQ_ERR_UNSUPPORTED
    assert rms_fused(D=mxq.MXQ_MAX_D + 32, ldx=mxq.MXQ_MAX_D + 32,
                     flags=mxq.MXQ_FLAG_FORCE_SPLIT) == mxq.MXQ_ERR_UNSUPPORTED
    assert rms_fused(D=mxq.MXQ_MAX_D + 32, ldx=mxq.MXQ_MAX_D + 32) == mxq.MXQ_ERR_UNSUPPORTED
    assert rms_fused(gamma=A8) == mxq.MXQ_ERR_ALIGN
    assert rms_fused(inv=A16 + 2) == mxq.MXQ_ERR_ALIGN


def test_rmsnorm_argument_errors():
    assert rms(eps=-1e-6) == mxq.MXQ_ERR_ARG
    assert rms(eps=float("nan")) == mxq.MXQ_ERR_ARG
    assert rms(eps=float("inf")) == mxq.MXQ_ERR_ARG
    assert rms(y=None) == mxq.MXQ_ERR_NULL
    assert rms(y=A8) == mxq.MXQ_ERR_ALIGN
    assert rms(gamma=A8) == mxq.MXQ_ERR_ALIGN


@pytest.mark.parametrize("call", [rms, cast])
def test_cast_flags_take_only_the_scale_rule(call):
    # the two-pass path and the plain cast have no variants to force
    assert call(flags=mxq.MXQ_FLAG_FORCE_REG) == mxq.MXQ_ERR_ARG
    assert call(flags=mxq.MXQ_FLAG_FORCE_LDS) == mxq.MXQ_ERR_ARG
    assert call(flags=mxq.MXQ_FLAG_FORCE_SPLIT) == mxq.MXQ_ERR_ARG
    assert call(flags=mxq.MXQ_FLAG_SCALE_CEIL | 16) == mxq.MXQ_ERR_ARG
    # the flag is validated after the shape: a bad shape still reports SHAPE
    assert call(D=0, flags=mxq.MXQ_FLAG_SCALE_CEIL) == mxq.MXQ_ERR_SHAPE


@pytest.mark.parametrize("call", [norm, rms, rms_fused, cast])
def test_empty_input_is_a_no_op(call):
    # T == 0 returns before any pointer is read or kernel launched
    assert call(T=0, x=None, codes=None, scales=None) == mxq.MXQ_OK


def test_torch_helpers_refuse_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mxq.mxnorm(x)
    with pytest.raises(TypeError):
        mxq.mxcast(x.float())


def test_caller_buffers_are_checked_before_any_launch():
    # a buffer of the wrong size, dtype or layout would be an out-of-bounds GPU
    # access, so the torch helpers refuse it on the host
    import torch
    cpu = torch.device("cpu")
    codes = torch.zeros(4, 64, dtype=torch.uint8)
    scales = torch.zeros(4, 2, dtype=torch.uint8)
    inv = torch.zeros(4, dtype=torch.float32)
    assert mxq._check_outputs((codes, scales, inv), 4, 64, mxq.MXQ_E4M3, cpu, True)[0] is codes
    with pytest.raises(ValueError):      # E2M1 packs two codes per byte: [4, 32]
        mxq._check_outputs((codes, scales, inv), 4, 64, mxq.MXQ_E2M1, cpu, True)
    with pytest.raises(ValueError):
        mxq._check_outputs((codes, scales[:, :1], inv), 4, 64, mxq.MXQ_E4M3, cpu, True)
    with pytest.raises(ValueError):
        mxq._check_outputs((codes, scales, inv.double()), 4, 64, mxq.MXQ_E4M3, cpu, True)
    with pytest.raises(ValueError):
        mxq._check_outputs((codes.t().contiguous().t(), scales, inv), 4, 64, mxq.MXQ_E4M3, cpu,
                           True)
    with pytest.raises(ValueError):
        mxq._check_outputs((codes,), 4, 64, mxq.MXQ_E4M3, cpu, True)
    with pytest.raises(ValueError):      # on another device than x
        mxq._check_outputs((codes, scales, inv), 4, 64, mxq.MXQ_E4M3, torch.device("meta"), True)
    mxq._check_gamma(None, 64, cpu)
    mxq._check_gamma(torch.ones(64, dtype=torch.bfloat16), 64, cpu)
    with pytest.raises(ValueError):
        mxq._check_gamma(torch.ones(64, dtype=torch.float32), 64, cpu)
    with pytest.raises(ValueError):
        mxq._check_gamma(torch.ones(128, dtype=torch.bfloat16)[::2], 64, cpu)


def test_product_path_does_not_touch_the_oracle():
    # the package and its sources never import or load the oracle
    pkg = os.path.join(ROOT, "norm_mx_quantisation_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text, f


def bwd(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, dy=A16, lddy=4096, inv=A16, T=8, D=4096, dx=A16,
             row_dot=None, dgamma=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return mxq.mxnorm_bwd(a["x"], a["ldx"], a["gamma"], a["dy"], a["lddy"], a["inv"], a["T"],
                          a["D"], a["dx"], a["row_dot"], a["dgamma"], a["ws"], a["wsb"],
                          a["stream"])


def test_backward_argument_errors():
    assert bwd(D=0) == mxq.MXQ_ERR_SHAPE
    assert bwd(D=4000 + 16) == mxq.MXQ_ERR_SHAPE
    assert bwd(T=-1) == mxq.MXQ_ERR_SHAPE
    assert bwd(ldx=2048) == mxq.MXQ_ERR_SHAPE
    assert bwd(lddy=2048) == mxq.MXQ_ERR_SHAPE
    assert bwd(D=8224, ldx=8224, lddy=8224) == mxq.MXQ_ERR_UNSUPPORTED
    assert bwd(x=None) == mxq.MXQ_ERR_NULL
    assert bwd(dy=None) == mxq.MXQ_ERR_NULL
    assert bwd(inv=None) == mxq.MXQ_ERR_NULL
    assert bwd(dx=None) == mxq.MXQ_ERR_NULL
    assert bwd(x=A8) == mxq.MXQ_ERR_ALIGN
    assert bwd(dy=A8) == mxq.MXQ_ERR_ALIGN
    assert bwd(dx=A8) == mxq.MXQ_ERR_ALIGN
    assert bwd(gamma=A8) == mxq.MXQ_ERR_ALIGN
    assert bwd(lddy=4100) == mxq.MXQ_ERR_ALIGN
    need = mxq.mxnorm_bwd_workspace_size(8, 4096)
    assert need >= 4096 * 4 * 2
    assert bwd(dgamma=A16, ws=None) == mxq.MXQ_ERR_NULL
    assert bwd(dgamma=A16, ws=A16, wsb=need - 1) == mxq.MXQ_ERR_ARG
    assert bwd(dgamma=A8, ws=A16, wsb=need) == mxq.MXQ_ERR_ALIGN
    assert bwd(dgamma=A16, ws=A8, wsb=need) == mxq.MXQ_ERR_ALIGN
    assert mxq.mxnorm_bwd_workspace_size(8, 100) == 0
    # empty input without dgamma launches nothing and reads no pointer
    assert bwd(T=0, x=None, dy=None, inv=None, dx=None) == mxq.MXQ_OK


def nbwd(**kw):
    a = dict(x=A16, ldx=4096, gamma=None, dy=A16, lddy=4096, inv=A16, T=8, D=4096, dx=A16,
             row_dot=None, dgamma=None, stream=None)
    a.update(kw)
    return mxq.mxnorm_bwd_noalloc(a["x"], a["ldx"], a["gamma"], a["dy"], a["lddy"], a["inv"],
                                  a["T"], a["D"], a["dx"], a["row_dot"], a["dgamma"], a["stream"])


def test_noalloc_backward_argument_errors():
    # the same checks as mxnorm_bwd, before any HIP call (these never reach the
    # scratch array's lookup or a launch)
    assert nbwd(D=0) == mxq.MXQ_ERR_SHAPE
    assert nbwd(T=-1) == mxq.MXQ_ERR_SHAPE
    assert nbwd(ldx=2048) == mxq.MXQ_ERR_SHAPE
    assert nbwd(D=8224, ldx=8224, lddy=8224) == mxq.MXQ_ERR_UNSUPPORTED
    assert nbwd(x=None) == mxq.MXQ_ERR_NULL
    assert nbwd(dx=None, dgamma=A16) == mxq.MXQ_ERR_NULL
    assert nbwd(x=A8) == mxq.MXQ_ERR_ALIGN
    assert nbwd(dgamma=A8) == mxq.MXQ_ERR_ALIGN
    assert nbwd(gamma=A8) == mxq.MXQ_ERR_ALIGN
    assert nbwd(lddy=4100) == mxq.MXQ_ERR_ALIGN


def test_backward_workspace_grows_slowly_with_rows():
    # one partial row of D floats per workgroup, at most 512 workgroups
    D = 4096
    small = mxq.mxnorm_bwd_workspace_size(64, D)
    big = mxq.mxnorm_bwd_workspace_size(1 << 20, D)
    assert small < big == 512 * D * 4


def gemm(**kw):
    a = dict(a=A16, lda=4096, sa=A16, ldsa=128, b=A16, ldb=4096, sb=A16, ldsb=128, M=256, N=256,
             K=4096, ea=0, eb=0, c=A16, ldc=256, ct=0, stream=None)
    a.update(kw)
    return mxq.mx_gemm(a["a"], a["lda"], a["sa"], a["ldsa"], a["b"], a["ldb"], a["sb"], a["ldsb"],
                       a["M"], a["N"], a["K"], a["ea"], a["eb"], a["c"], a["ldc"], a["ct"],
                       a["stream"])


def test_gemm_argument_errors():
    assert gemm(K=0) == mxq.MXQ_ERR_SHAPE
    assert gemm(K=100) == mxq.MXQ_ERR_SHAPE
    assert gemm(M=-1) == mxq.MXQ_ERR_SHAPE
    assert gemm(lda=2048) == mxq.MXQ_ERR_SHAPE
    assert gemm(ldsb=64) == mxq.MXQ_ERR_SHAPE
    assert gemm(ldc=100) == mxq.MXQ_ERR_SHAPE
    assert gemm(ea=3) == mxq.MXQ_ERR_ARG
    assert gemm(ct=2) == mxq.MXQ_ERR_ARG
    # packed E2M1 rows hold K / 2 bytes: lda = 2048 passes the shape check
    assert gemm(ea=1, lda=2047) == mxq.MXQ_ERR_SHAPE
    assert gemm(ea=1, lda=2048, a=None) == mxq.MXQ_ERR_NULL
    assert gemm(eb=1, ldb=2048, b=None) == mxq.MXQ_ERR_NULL
    assert gemm(eb=1, ldb=2032) == mxq.MXQ_ERR_SHAPE
    assert gemm(K=160, lda=160, ldb=160, ldsa=8, ldsb=8) == mxq.MXQ_ERR_UNSUPPORTED  # K % 128
    assert gemm(a=None) == mxq.MXQ_ERR_NULL
    assert gemm(c=None) == mxq.MXQ_ERR_NULL
    assert gemm(a=A8) == mxq.MXQ_ERR_ALIGN
    assert gemm(lda=4104) == mxq.MXQ_ERR_ALIGN
    assert gemm(ldsa=130) == mxq.MXQ_ERR_ALIGN
    assert gemm(c=A16 + 2) == mxq.MXQ_ERR_ALIGN            # fp32 output needs 4-byte alignment
    assert gemm(M=0, a=None, sa=None, b=None, sb=None, c=None) == mxq.MXQ_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU fallback: without the built library every call raises
    monkeypatch.setattr(mxq, "_lib", None)
    monkeypatch.setattr(mxq, "LIB_PATH", str(tmp_path / "libmxq.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mxq.lib()
    with pytest.raises(RuntimeError, match="not built"):
        mxq.mxq_abi_version()


def test_mx_views_are_the_torch_float8_and_float4_types():
    # the binding's dtype views of the uint8 outputs decode to the format values
    import torch
    codes = torch.tensor([[0x38, 0xB8, 0x7E, 0x01]], dtype=torch.uint8)
    scales = torch.tensor([[127, 130]], dtype=torch.uint8)
    cv, sv = mxq.mx_views(codes, scales, "e4m3")
    assert cv.dtype == torch.float8_e4m3fn and sv.dtype == torch.float8_e8m0fnu
    assert cv.float().tolist() == [[1.0, -1.0, 448.0, 2.0 ** -9]]
    assert sv.float().tolist() == [[1.0, 8.0]]
    packed = torch.tensor([[0x72, 0x0F]], dtype=torch.uint8)   # (1.0, 6.0), (-6.0, 0.0)
    cv, _ = mxq.mx_views(packed, scales, "e2m1")
    assert cv.dtype == torch.float4_e2m1fn_x2
    nv = torch.tensor([[0x38]], dtype=torch.uint8)
    _, sv = mxq.mx_views(packed, nv, "nvfp4")
    assert sv.dtype == torch.float8_e4m3fn and sv.float().item() == 1.0
    with pytest.raises(ValueError):
        mxq.mx_views(codes, scales, "e5m2")

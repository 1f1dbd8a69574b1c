"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/mxq_oracle.c) is compiled with gcc and the sanitizers into
  a drive (tests/helpers/oracle_sanitize_main.c) that calls every entry point
  with exact-size heap buffers: both formats, roundings and scale rules, every
  p, strided rows, special values, both oracle modes, NVFP4, the backward, the
  MX GEMM and the invalid-argument statuses. A build of the same drive with one
  buffer a byte short must be reported, so the check is known to be live.
- The library's host code (argument validation and status codes of every C-ABI
  entry point, before any HIP call) is compiled with the sanitizers on the host
  pass only (the device code is built as usual and never runs) and driven by
  tests/helpers/abi_sanitize_main.cpp, without a GPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HELPERS = os.path.join(ROOT, "tests", "helpers")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"   # the drive and the link: the compiler hipcc drives
ROCM_LIB = "/opt/rocm/lib"
SAN_ENV = dict(os.environ,
               ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
GCC_SAN = ["-O1", "-g", "-fno-fast-math", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all"]


def _gcc_oracle_drive(tmp_path, name, extra=()):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / name)
    subprocess.run(["gcc", *GCC_SAN, *extra, "-o", exe,
                    os.path.join(HELPERS, "oracle_sanitize_main.c"), "-lm"],
                   check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    r = _gcc_oracle_drive(tmp_path, "oracle_san")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitizer drive: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_drive_reports_a_planted_short_buffer(tmp_path):
    r = _gcc_oracle_drive(tmp_path, "oracle_san_planted", ["-DMXQ_PLANT_SHORT_SCALES"])
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    if not os.path.exists(HIPCC) or not os.path.exists(CLANGXX):
        pytest.skip("hipcc or ROCm's clang++ not found")
    inc = os.path.join(ROOT, "include")
    csrc = os.path.join(ROOT, "norm_mx_quantisation_amd", "csrc")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-I", inc]
    procs, objs = [], []
    for src in ("mxq.hip", "mxq_bwd.hip", "mx_gemm.hip"):
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", "-o", obj, os.path.join(csrc, src)],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    main_obj = str(tmp_path / "abi_main.o")
    procs.append(subprocess.Popen(
        [CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I", inc, "-c", "-o", main_obj,
         os.path.join(HELPERS, "abi_sanitize_main.cpp")],
        stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-4000:]
    exe = str(tmp_path / "abi_san")
    subprocess.run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, main_obj, *objs,
                    "-L", ROCM_LIB, "-lamdhip64", "-Wl,-rpath," + ROCM_LIB],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "abi sanitizer drive: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr

"""Build libmxq.so (the HIP kernels and C ABI) and libmxq_floor.so (the
bytes-only reference kernels the timing module runs beside it) in-tree for
gfx950."""

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("mxq.hip", "mxq_bwd.hip", "mx_gemm.hip")]
DEV_HDR = os.path.join(PKG, "csrc", "mxq_device.h")
HDR = os.path.join(ROOT, "include", "mxq.h")
LIB = os.path.join(PKG, "libmxq.so")
FLOOR_SRC = os.path.join(PKG, "csrc", "stream_floor.hip")
FLOOR_LIB = os.path.join(PKG, "libmxq_floor.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # the arithmetic order is the one written in the source: no contraction
    "-ffp-contract=off",
    # packed-fp32 VALU ops stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _stale(lib, deps):
    return not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(p) for p in deps)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile both libraries (each source in its own hipcc process, all in
    parallel) and return the path of libmxq.so. Without force, only a library
    older than its sources is rebuilt."""
    jobs = []
    if force or _stale(LIB, SRCS + [HDR, DEV_HDR]):
        jobs.append((LIB, SRCS))
    if force or _stale(FLOOR_LIB, [FLOOR_SRC, DEV_HDR]):
        jobs.append((FLOOR_LIB, [FLOOR_SRC]))
    if not jobs:
        return LIB
    with tempfile.TemporaryDirectory() as tmpdir:
        objs, procs = {}, []
        for lib, srcs in jobs:
            for src in srcs:
                obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
                cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, src]
                if verbose:
                    print(" ".join(cmd), file=sys.stderr)
                procs.append(subprocess.Popen(cmd, cwd=tmpdir, stdout=subprocess.PIPE,
                                              stderr=subprocess.PIPE, text=True))
                objs.setdefault(lib, []).append(obj)
        errors = []
        for p in procs:
            out, err = p.communicate()
            if p.returncode != 0:
                errors.append(out + err)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        for lib, _ in jobs:
            tmp = lib + ".tmp"
            cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs[lib]]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            res = subprocess.run(cmd, cwd=tmpdir, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
            os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))

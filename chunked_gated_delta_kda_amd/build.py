"""Build libkda.so (the gfx950 HIP library behind include/kda.h) in-tree.

    python -m chunked_gated_delta_kda_amd.build

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32
instruction selection disabled, and linked into chunked_gated_delta_kda_amd/libkda.so.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_split.hip", "kda_h32.hip", "kda_fused.hip", "kda_recurrent.hip", "kda_bwd.hip"]

COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Werror",
          "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: the state is also touched by VALU every chunk,
          # and the AGPR form costs a copy per element each way
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I" + INCLUDE, "-I" + CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda.so)")


def _compile(src, extra=()):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{_filter(r.stderr)}")
    return obj


def _filter(err):
    # the host pass does not know the packed-fp32 target feature; that note is harmless
    return "\n".join(x for x in err.splitlines() if "packed-fp32-ops" not in x)


def build(verbose=False, extra=(), out=None):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{_filter(r.stderr)}")
    os.replace(tmp, lib)
    if verbose:
        print(lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    out = None
    if "-o" in args:
        i = args.index("-o")
        out = os.path.abspath(args[i + 1])
        del args[i:i + 2]
    build(verbose=True, extra=tuple(args), out=out)

"""Build the oracle's shared library (test infrastructure only).

Compiles oracle/kda_oracle.c with the host C compiler into
oracle/libkda_oracle.so. Nothing here touches the GPU or the HIP sources.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")          # forward
SRC_BWD = os.path.join(HERE, "kda_oracle_bwd.c")  # backward (gradients of the forward)
LIB = os.path.join(HERE, "libkda_oracle.so")


def compile_oracle(src=SRC, out=LIB, cc=None, extra=(), strict=True):
    """Compile ``src`` (a path or a list of paths) into the shared library ``out``; returns ``out``."""
    cc = cc or os.environ.get("CC", "gcc")
    tmp = out + ".tmp"
    warn = ["-Wall", "-Wextra", "-Werror"] if strict else ["-w"]
    srcs = [src] if isinstance(src, str) else list(src)
    cmd = [cc, "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", *warn, *extra, *srcs, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build():
    return compile_oracle([SRC, SRC_BWD])


if __name__ == "__main__":
    print(compile_oracle(*sys.argv[1:2]))

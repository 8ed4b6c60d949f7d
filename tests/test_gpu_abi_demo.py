"""The library through its C ABI alone: tests/abi_demo.c (plain C, HIP runtime API,
include/kda.h; no Python binding, no torch) runs a packed prefill and a decode step
on the GPU and checks them against the oracle's C library."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "abi_demo_bin")


def test_c_abi_demo():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BIN):      # built by __graft_entry__.build(); host compiler only
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__._build_abi_demo()
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, file=sys.stderr, flush=True)
    assert r.returncode == 0 and "PASS" in r.stdout, r.stdout + r.stderr

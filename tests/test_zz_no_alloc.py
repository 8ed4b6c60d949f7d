"""kda_fwd_noalloc through the C ABI against kda_fwd_ex with the same variant (the
existing entry point whose kernels it shares), on two calls in a row, the second with
a smaller input: the fixed per-device scratch keeps the first call's contents, which
the second must not read. Both are also held to the oracle gate."""
import ctypes
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth
from kda_check import compare, run_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(fn_name, w, variant=None):
    import torch
    from chunked_gated_delta_kda_amd import native

    lib = native.load_library()
    d = synth.to_device(w)
    out = torch.full((w.T, w.H, 128), float("nan"), device="cuda")
    fin = torch.full((w.N, w.H, 128, 128), float("nan"), device="cuda")
    st = torch.cuda.current_stream()
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    args = [p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), d["scale"], p(d["cu_seqlens"]),
            w.N, w.T, w.H, 128, p(d["initial_state"]), p(out), p(fin), ctypes.c_void_p(st.cuda_stream)]
    if fn_name == "kda_fwd_noalloc":
        rc = lib.kda_fwd_noalloc(*args)
    else:
        opt = native.KdaOptions(variant=native.VARIANTS[variant])
        rc = lib.kda_fwd_ex(*args, ctypes.byref(opt))
    torch.cuda.synchronize()
    assert rc == 0, native.status_string(rc)
    return out.cpu().numpy(), fin.cpu().numpy()


# (lengths, H, seed): the second call of each pair is smaller (fewer sequences, tokens
# and heads); the last pair's second call is short enough for the token loop
PAIRS = [
    (([300, 0, 129, 700, 17], 3, 41), ([40, 9], 2, 42)),
    (([1024] * 8, 4, 43), ([2, 1, 3], 1, 44)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["varlen", "uniform_then_tiny"])
def test_noalloc_matches_fwd_ex(pair):
    import chunked_gated_delta_kda_amd as kda

    for lengths, H, seed in pair:
        w = synth.make_workload(lengths, H, seed, with_initial_state=True, clamp_frac=0.1)
        variant = kda.select_variant(w.N, w.T, w.H)
        variant = "recurrent" if variant == "recurrent" else "fused"
        _say(f"[noalloc] lengths={lengths} H={H} -> {variant}")
        o1, f1 = _call("kda_fwd_noalloc", w)
        o2, f2 = _call("kda_fwd_ex", w, variant)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(f1, f2)
        ro, rf = run_oracle(w)
        ok, mo, mf = compare(w, o1, f1, ro, rf)
        _say(f"  o {mo}\n  S {mf}")
        assert ok


def test_noalloc_rejects_too_many_sequences():
    import torch
    from chunked_gated_delta_kda_amd import native

    lib = native.load_library()
    N = native.NOALLOC_MAX_SEQS + 1
    T, H = 4 * N, 1
    # the size check comes before any pointer is used or anything is enqueued
    dummy = torch.empty(16, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    rc = lib.kda_fwd_noalloc(p, p, p, p, p, 0.1, p, N, T, H, 128, None, p, None, None)
    assert native.STATUS[rc] == "KDA_ERR_SCRATCH"

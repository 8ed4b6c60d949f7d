"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from chunked_gated_delta_kda_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(native.LIB_PATH):
        pytest.skip("libkda.so not built")
    return native.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(native.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.kda_version()
    for s in range(8):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation first


def call(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, scale=0.088, cu=P, N=1, T=16, H=2, D=128, s0=None,
             out=P, fin=P, opt=None)
    a.update(over)
    opt = ctypes.byref(a["opt"]) if a["opt"] is not None else None
    return lib.kda_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], a["N"],
                          a["T"], a["H"], a["D"], a["s0"], a["out"], a["fin"], None, opt)


def test_validation_errors(lib):
    assert call(lib, D=64) == 3                       # KDA_ERR_UNSUPPORTED
    assert call(lib, scale=float("nan")) == 3
    assert call(lib, scale=float("inf")) == 3
    assert call(lib, N=0) == 2                        # KDA_ERR_SHAPE
    assert call(lib, T=-1) == 2
    assert call(lib, H=0) == 2
    assert call(lib, cu=None, N=2) == 2
    assert call(lib, q=None) == 1                     # KDA_ERR_NULL
    assert call(lib, beta=None) == 1
    assert call(lib, out=None) == 1
    opts = lambda **kw: native.KdaOptions(**{"variant": 0, "n_stage_events": 0, **kw})
    assert call(lib, opt=opts(variant=7)) == 3
    assert call(lib, opt=opts(n_stage_events=1)) == 3                         # 1 stage event
    assert call(lib, opt=opts(n_stage_events=4)) == 3                         # events NULL
    assert call(lib, opt=opts(reserved=1)) == 3                               # reserved != 0
    assert call(lib, opt=opts(g_dtype=2)) == 3                                # unknown g dtype
    assert call(lib, opt=opts(state_dtype=-1)) == 3                           # unknown state dtype
    # bf16 g or states: the fused variant does not read them
    assert call(lib, opt=opts(variant=2, g_dtype=1)) == 3
    assert call(lib, opt=opts(variant=2, state_dtype=1)) == 3
    small = opts(variant=1, workspace=ctypes.c_void_p(256), workspace_bytes=10)
    assert call(lib, opt=small) == 4                  # KDA_ERR_ALLOC: workspace too small
    small.g_dtype = 1                                 # still too small with bf16 g (forms 401/402)
    assert call(lib, opt=small) == 4
    # final_state partially overlapping initial_state (as fp32, and as bf16 states)
    assert call(lib, s0=ctypes.c_void_p(4096), fin=ctypes.c_void_p(4096 + 64)) == 7
    n_bf16 = 2 * 128 * 128 * 2
    assert call(lib, s0=ctypes.c_void_p(4096), fin=ctypes.c_void_p(4096 + n_bf16 - 64),
                opt=opts(state_dtype=1, variant=1, workspace=ctypes.c_void_p(256), workspace_bytes=10)) == 7


def decode_call(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, scale=0.088, N=4, H=2, D=128, s_in=None, s_out=P, out=P)
    a.update(over)
    return lib.kda_decode(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["N"], a["H"],
                          a["D"], a["s_in"], a["s_out"], a["out"], None)


def test_decode_validation_errors(lib):
    assert decode_call(lib, D=64) == 3
    assert decode_call(lib, scale=float("nan")) == 3
    assert decode_call(lib, N=0) == 2
    assert decode_call(lib, H=0) == 2
    assert decode_call(lib, q=None) == 1
    assert decode_call(lib, g=None) == 1
    assert decode_call(lib, out=None) == 1
    assert decode_call(lib, s_in=ctypes.c_void_p(4096), s_out=ctypes.c_void_p(4096 + 64)) == 7


def test_decode_ex_validation_errors(lib):
    def call_ex(dtype, s_in=None, s_out=P, N=4, D=128):
        return lib.kda_decode_ex(P, P, P, P, P, 0.088, N, 2, D, s_in, s_out, P, None, dtype)
    assert call_ex(2) == 3                                       # unknown state dtype
    assert call_ex(-1) == 3
    assert call_ex(1, D=64) == 3
    assert call_ex(1, N=0) == 2
    # bf16 states are half as long: these two overlap by 64 bytes only as bf16
    n_bf16 = 4 * 2 * 128 * 128 * 2
    assert call_ex(1, s_in=ctypes.c_void_p(4096), s_out=ctypes.c_void_p(4096 + n_bf16 - 64)) == 7


def test_workspace_bytes(lib):
    assert lib.kda_workspace_bytes(0, 16, 1, 1) == 0
    b = lib.kda_workspace_bytes(1, 8192, 32, 1)
    assert b >= (8192 // 32) * 32 * 37888     # one 32-token record per chunk-head
    assert lib.kda_select_variant(1, 8192, 32) in (1, 2, 3)
    assert lib.kda_workspace_bytes(1, 8192, 32, 3) == 0    # the recurrent variant needs none


def test_launch_plan():
    from chunked_gated_delta_kda_amd import native as nat
    for N, T, H in ((1, 8192, 32), (2, 4096, 8), (8, 8192, 16), (64, 100000, 32), (12, 32768, 32),
                    (200, 51200, 8)):
        plan = nat.launch_plan(N, T, H, "split")
        kinds = [p[0] for p in plan]
        # the 32-token forms form the chunk map in their first prep for up to 63
        # sequences; otherwise it is a launch of its own
        head = ["prep"] if N <= 63 and plan[0][3] == 32 else ["chunk_map", "prep"]
        assert kinds[:len(head)] == head and kinds[-1] == "recur"
        assert set(kinds[len(head):-1]) <= {"recur_prep"}
        cl = plan[0][3]
        assert cl in (16, 32) and all(p[3] == cl for p in plan)
        one = nat.SEGMENT_ONE
        assert f"#define KDA_SEGMENT_ONE {one}" in open(HEADER).read()
        # the prep segments and the recurrence segments each tile [0, SEGMENT_ONE) in
        # order, and a segment's records are prepared in an earlier launch than its
        # recurrence
        work = plan[len(head) - 1:]      # the launches after the chunk map, if any
        preps = [p[1] for p in work if p[1] != (0, 0)]
        recs = [p[2] for p in work if p[2] != (0, 0)]
        for ranges in (preps, recs):
            assert ranges[0][0] == 0 and ranges[-1][1] == one
            assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
            assert all(a < b for a, b in ranges)
        for i, p in enumerate(plan):
            if p[2] != (0, 0):
                lo, hi = p[2]
                covered = [q[1] for q in plan[:i] if q[1] != (0, 0)]
                assert any(a <= lo for a, _ in covered) and max(b for _, b in covered) >= hi
        # of a sequence of any length, the recurrence segments take each chunk once
        for c in (0, 1, 2, 7, 64, 513, 4096):
            got = []
            for lo, hi in recs:
                got += range(c * lo // one, c * hi // one)
            assert got == list(range(c))
    # few long chains: the recurrence runs over parts of each sequence, in one launch
    # entry after the prep of all chunks
    assert [p[0] for p in nat.launch_plan(1, 65536, 8, "split")] == ["prep", "parts"]
    assert [p[0] for p in nat.launch_plan(1, 65536, 4, "split")] == ["prep", "parts"]
    assert [p[0] for p in nat.launch_plan(1, 8192, 8, "split")] == ["prep", "parts"]
    assert [p[0] for p in nat.launch_plan(1, 2048, 8, "split")] == ["prep", "recur"]
    # 16 chains of 1,024 chunks (32 tokens) each: four parts, pass 2 with two slices per block
    assert [p[0] for p in nat.launch_plan(2, 65536, 8, "split")] == ["prep", "parts"]
    assert [p[0] for p in nat.launch_plan(1, 32768, 16, "split")][-1] == "parts"   # four, two-slice pass 2
    assert [p[0] for p in nat.launch_plan(1, 8192, 16, "split")][-1] == "parts"    # four parts of 64 chunks
    assert [p[0] for p in nat.launch_plan(1, 8192, 32, "split")][-1] != "parts"    # two parts do not pay
    assert [p[0] for p in nat.launch_plan(1, 4096, 4, "split")][-1] != "parts"     # parts under 64 chunks
    # many chains (the two-slice 32-token form, or the per-chain hybrid) run whole by default
    assert [p[0] for p in nat.launch_plan(12, 32768, 32, "split")] == ["prep", "recur"]
    # the per-chain hybrid (16-token records) of many short sequences keeps the chunk-map launch
    assert [p[0] for p in nat.launch_plan(200, 51200, 8, "split")] == ["chunk_map", "prep", "recur"]
    assert [p[0] for p in nat.launch_plan(8, 8192, 16, "fused")] == ["chunk_map", "fused"]
    assert nat.launch_plan(0, 16, 1, "split") == []
    assert [p[0] for p in nat.launch_plan(8, 8192, 16, "recurrent")] == ["recurrent"]


def bwd_call(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, scale=0.088, cu=P, N=1, T=16, H=2, D=128, s0=None, do=P,
             dsf=None, dq=P, dk=P, dv=P, dg=P, db=P, ds0=None, ws=ctypes.c_void_p(256), wsb=10)
    a.update(over)
    return lib.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], a["N"], a["T"],
                       a["H"], a["D"], a["s0"], a["do"], a["dsf"], a["dq"], a["dk"], a["dv"], a["dg"],
                       a["db"], a["ds0"], None, a["ws"], a["wsb"])


def test_bwd_validation_errors(lib):
    assert bwd_call(lib, D=64) == 3
    assert bwd_call(lib, scale=float("nan")) == 3
    assert bwd_call(lib, N=0) == 2
    assert bwd_call(lib, T=-1) == 2
    assert bwd_call(lib, cu=None, N=2) == 2
    for name in ("q", "g", "beta", "do", "dq", "dk", "dv", "dg", "db"):
        assert bwd_call(lib, **{name: None}) == 1, name
    assert bwd_call(lib) == 4                         # workspace too small


def test_bwd_workspace_bytes(lib):
    assert lib.kda_bwd_workspace_bytes(0, 16, 1) == 0
    N, T, H = 8, 8192, 16
    state = 128 * 128 * 4
    b = lib.kda_bwd_workspace_bytes(N, T, H)
    # a state per block of KDA_BWD_BLOCK tokens and head
    assert b >= (T // 4) * H * state
    assert "#define KDA_BWD_BLOCK 4" in open(HEADER).read()


def test_bwd_workspace_forms(lib, monkeypatch):
    """The workspace covers each backward form: the checkpoints alone (two 8-wave blocks per
    chain, no parts); plus four partial sums of 385 floats per token-head (four 4-wave
    blocks per chain, below 96 chains); plus four states per part slot and head and the
    parts' offsets (over parts)."""
    state = 128 * 128 * 4
    N, T, H = 1, 8192, 32
    for var in ("KDA_BWD_WAVES", "KDA_BWD_PARTS", "KDA_BWD_PART_TOKENS"):
        monkeypatch.delenv(var, raising=False)
    monkeypatch.setenv("KDA_BWD_WAVES", "8")
    monkeypatch.setenv("KDA_BWD_PARTS", "1")
    base = lib.kda_bwd_workspace_bytes(N, T, H)
    assert base >= (T // 4) * H * state
    monkeypatch.setenv("KDA_BWD_WAVES", "4")
    partial = lib.kda_bwd_workspace_bytes(N, T, H)
    assert partial - base >= 4 * T * H * 385 * 4
    monkeypatch.setenv("KDA_BWD_PARTS", "8")
    parts = lib.kda_bwd_workspace_bytes(N, T, H)
    assert parts - partial >= 4 * N * 8 * H * state + 2 * (N * 8 + 1) * 4
    # the default for one long sequence of 32 heads: four-wave blocks over parts
    monkeypatch.delenv("KDA_BWD_WAVES")
    monkeypatch.delenv("KDA_BWD_PARTS")
    assert lib.kda_bwd_workspace_bytes(N, T, H) == parts

"""Malformed cu_seqlens on the GPU: every variant sanitises the offsets (clamped to
[0, T], each raised to the largest offset before it) before using them, raises the device
error bit 2 (in the device error word, and in the workspace's error word where there is a
workspace), and the call completes with every access in bounds. Ranges that were valid
keep correct outputs."""
import sys

import numpy as np
import pytest

import oracle
from chunked_gated_delta_kda_amd import synth
from kda_check import run_oracle

pytestmark = pytest.mark.gpu

ERR_CU_SEQLENS = 2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, cu, variant):
    """One call with the given offsets; returns (o, final state, workspace error word or
    None for the variant without a workspace, device error word)."""
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    d = synth.to_device(w)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    N = len(cu) - 1
    nbytes = kda.workspace_bytes(N, w.T, w.H, variant)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    out = torch.full((w.T, w.H, 128), 7.0, device="cuda")
    kda.device_errors(clear=True)
    o, f = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], cu_t, None, variant=variant,
                   workspace=ws, out=out)
    dev_err = kda.device_errors(clear=True)
    word = None
    if ws is not None:
        off = native.error_word_offset(N)
        word = int(ws[off:off + 4].view(torch.int32).item())
    return o.cpu().numpy(), f.cpu().numpy(), word, dev_err


# (offsets, T): decreasing, past T, negative start, nonzero start, short of T
CASES = [([0, 50, 30, 100], 100), ([0, 60, 140], 100), ([-5, 40, 100], 100), ([7, 40, 100], 100),
         ([0, 30, 70], 100), ([0, 100, 0, 100], 100)]


def _many(n):
    """n sequences over 100 tokens (many empty), one offset decreasing and one past T:
    63 is the most the first prep's wave-held chunk map takes, 64 the fewest the
    chunk-map launch does."""
    rng = np.random.Generator(np.random.PCG64(n))
    cu = np.sort(rng.integers(0, 101, size=n + 1))
    cu[0], cu[-1] = 0, 100
    cu[10] = cu[9] - 5
    cu[40] = 140
    return [int(x) for x in cu], 100


CASES += [_many(63), _many(64)]


@pytest.mark.parametrize("variant", ["split", "fused", "recurrent"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c[0])) if len(c[0]) < 8 else f"N{len(c[0]) - 1}")
def test_malformed_cu_seqlens(case, variant):
    cu, T = case
    w = synth.make_workload([T], 2, 5)
    _say(f"[robust] cu_seqlens={cu} T={T} variant={variant}")
    o, f, word, dev_err = _run(w, cu, variant)
    assert dev_err == ERR_CU_SEQLENS
    assert word in (None, ERR_CU_SEQLENS)
    # sanitised offsets as the chunk map forms them
    cs = np.maximum.accumulate(np.clip(np.asarray(cu), 0, T))
    covered = np.zeros(T, dtype=bool)
    for a, b in zip(cs[:-1], cs[1:]):
        covered[a:b] = True
    assert np.isfinite(o[covered]).all() and np.isfinite(f).all()
    assert (o[~covered] == 7.0).all()          # rows of no sequence are left untouched
    # each sanitised sequence is a valid sequence: its outputs match the oracle
    lens = np.diff(cs)
    sub = synth.Workload(name="sub", q=w.q[cs[0]:cs[-1]], k=w.k[cs[0]:cs[-1]], v=w.v[cs[0]:cs[-1]],
                         g=w.g[cs[0]:cs[-1]], beta=w.beta[cs[0]:cs[-1]],
                         cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    ro, rf = run_oracle(sub)
    mo = synth.parity(o[cs[0]:cs[-1]], ro)
    mf = synth.parity(f, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert synth.passes(mo) and synth.passes(mf)


@pytest.mark.parametrize("variant", ["split", "fused", "recurrent"])
def test_wellformed_raises_nothing(variant):
    w = synth.make_workload([30, 70], 2, 6)
    o, f, word, dev_err = _run(w, [0, 30, 100], variant)
    assert dev_err == 0 and word in (None, 0)


def test_plain_kda_fwd_reports_malformed_offsets():
    """kda_fwd without options (the library allocates and frees its own workspace): the
    error is still visible through the device error word."""
    import ctypes
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    lib = native.load_library()
    w = synth.make_workload([100], 2, 8)
    d = synth.to_device(w)
    for cu, expect in (([0, 60, 30, 100], ERR_CU_SEQLENS), ([0, 30, 100], 0)):
        cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
        out = torch.empty((w.T, w.H, 128), device="cuda")
        fin = torch.empty((len(cu) - 1, w.H, 128, 128), device="cuda")
        kda.device_errors(clear=True)
        st = torch.cuda.current_stream()
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = lib.kda_fwd(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), d["scale"], p(cu_t),
                         len(cu) - 1, w.T, w.H, 128, None, p(out), p(fin), ctypes.c_void_p(st.cuda_stream))
        assert rc == 0
        bits = kda.device_errors(clear=True)
        _say(f"[robust] plain kda_fwd cu={cu}: device error bits {bits}")
        assert bits == expect
        # Python fwd with check=True raises on the same offsets
        if expect:
            with pytest.raises(native.KdaDeviceError):
                kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], cu_t, check=True)
        else:
            kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], cu_t, check=True)


@pytest.mark.parametrize("waves", ["8", "4"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c[0])))
def test_bwd_malformed_cu_seqlens(monkeypatch, case, waves):
    """The backward sanitises offsets as the forward does: the error bit is raised; every
    sanitised sequence's gradients match the oracle on that sequence; rows of no sequence
    get zero dq, dk, dg and dbeta. Both workgroup forms."""
    import torch
    import chunked_gated_delta_kda_amd as kda

    monkeypatch.setenv("KDA_BWD_WAVES", waves)
    cu, T = case
    w = synth.make_workload([T], 2, 15, clamp_frac=0.1)
    rng = np.random.Generator(np.random.PCG64(16))
    do = rng.standard_normal((T, w.H, 128)).astype(np.float32)
    _say(f"[robust] backward cu_seqlens={cu} T={T} waves={waves}")
    d = synth.to_device(w)
    cs = np.maximum.accumulate(np.clip(np.asarray(cu), 0, T))
    N = len(cu) - 1
    dsf = rng.standard_normal((N, w.H, 128, 128)).astype(np.float32) * np.float32(0.1)
    kda.device_errors(clear=True)
    gr = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], torch.from_numpy(do).cuda(), d["scale"],
                 torch.tensor(cu, dtype=torch.int32, device="cuda"), None, torch.from_numpy(dsf).cuda())
    torch.cuda.synchronize()
    assert kda.device_errors(clear=True) == ERR_CU_SEQLENS
    got = {n: gr[n].cpu().numpy() for n in ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")}
    covered = np.zeros(T, dtype=bool)
    for a, b in zip(cs[:-1], cs[1:]):
        covered[a:b] = True
    for n in ("dq", "dk", "dg", "dbeta"):
        assert (got[n][~covered] == 0.0).all(), n
    lens = np.diff(cs)
    sub = synth.Workload(name="sub", q=w.q[cs[0]:cs[-1]], k=w.k[cs[0]:cs[-1]], v=w.v[cs[0]:cs[-1]],
                         g=w.g[cs[0]:cs[-1]], beta=w.beta[cs[0]:cs[-1]],
                         cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    ref = oracle.kda_backward(**synth.oracle_inputs(sub), d_out=do[cs[0]:cs[-1]], d_final_state=dsf)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        m = synth.parity(got[n][cs[0]:cs[-1]], ref[n])
        assert synth.passes(m), (n, m)
    m = synth.parity(got["d_initial_state"], ref["d_initial_state"])
    assert synth.passes(m), ("d_initial_state", m)

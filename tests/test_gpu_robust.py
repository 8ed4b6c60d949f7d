"""Malformed cu_seqlens on the GPU: the chunk map sanitises the offsets (clamped to
[0, T], made non-decreasing) before any other kernel reads them, sets the device error
word to 2, and the call completes with every access in bounds. Ranges that were valid
keep correct outputs."""
import sys

import numpy as np
import pytest

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
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    d = synth.to_device(w)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    N = len(cu) - 1
    nbytes = kda.workspace_bytes(N, w.T, w.H, variant)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((w.T, w.H, 128), 7.0, device="cuda")
    o, f = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], cu_t, None, variant=variant,
                   workspace=ws, out=out)
    torch.cuda.synchronize()
    off = native.error_word_offset(N)
    return o.cpu().numpy(), f.cpu().numpy(), int(ws[off:off + 4].view(torch.int32).item())


# (offsets, T): decreasing, past T, negative start, nonzero start, short of T
CASES = [([0, 50, 30, 100], 100), ([0, 60, 140], 100), ([-5, 40, 100], 100), ([7, 40, 100], 100),
         ([0, 30, 70], 100), ([0, 100, 0, 100], 100)]


@pytest.mark.parametrize("variant", ["split", "fused"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c[0])))
def test_malformed_cu_seqlens(case, variant):
    cu, T = case
    w = synth.make_workload([T], 2, 5)
    _say(f"[robust] cu_seqlens={cu} T={T} variant={variant}")
    o, f, err = _run(w, cu, variant)
    assert err == ERR_CU_SEQLENS
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


def test_wellformed_clears_error_word():
    w = synth.make_workload([30, 70], 2, 6)
    o, f, err = _run(w, [0, 30, 100], "split")
    assert err == 0

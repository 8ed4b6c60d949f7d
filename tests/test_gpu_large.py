"""GPU parity past 32-bit element offsets.

A batch of two sequences, 64 heads: a 299,000-token prefix sequence and a
1,000-token sequence behind it, so that every input and output element of the
second sequence lies beyond 2^31 elements (and its chunk records beyond 2^32
bytes). The second sequence is drawn by the seeded generator and checked
against the fp64 oracle, output and final state, to the parity gate; the prefix
repeats that sequence's inputs, and its outputs and final state are checked to
be finite. Every kernel family runs: the default split path, the segmented
path, the per-chain hybrid, the 32-token chunks, the fused kernel and the token
loop.
"""
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth
from kda_check import compare, run_oracle

pytestmark = pytest.mark.gpu

H = 64
REPS = 299
LAST = 1000
L0 = REPS * LAST
D = synth.HEAD_DIM

CASES = [
    ("split", {}),
    ("split", {"KDA_RECUR_WAVES": "101", "KDA_SEGMENTS": "3"}),
    ("split", {"KDA_RECUR_WAVES": "9"}),
    ("split", {"KDA_RECUR_WAVES": "9", "KDA_SEGMENTS": "3"}),
    ("split", {"KDA_PARTS": "3"}),
    ("split", {"KDA_RECUR_WAVES": "401", "KDA_SEGMENTS": "2"}),
    ("fused", {}),
    ("recurrent", {}),
]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def batch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert L0 * H * D > 2 ** 31
    w = synth.make_workload([LAST], H, 4242, with_initial_state=True, clamp_frac=0.05)
    ref = run_oracle(w)
    blk = synth.to_device(w)
    T = L0 + LAST
    dev = {}
    for name in ("q", "k", "v", "g", "beta"):
        x = blk[name]
        full = torch.empty((T,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
        full[:L0].view((REPS,) + tuple(x.shape)).copy_(x.unsqueeze(0).expand((REPS,) + tuple(x.shape)))
        full[L0:].copy_(x)
        dev[name] = full
    dev["cu_seqlens"] = torch.tensor([0, L0, T], dtype=torch.int32, device="cuda")
    s0 = torch.zeros((2, H, D, D), dtype=torch.float32, device="cuda")
    s0[1].copy_(blk["initial_state"][0])
    dev["initial_state"] = s0
    torch.cuda.synchronize()
    yield w, ref, dev, blk["scale"]
    dev.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant,env", CASES,
                         ids=["-".join([c[0]] + [f"{k[4:].lower()}{v}" for k, v in c[1].items()]) for c in CASES])
def test_offsets_past_2_31(batch, variant, env, monkeypatch):
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    w, (ro, rf), d, scale = batch
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    T = L0 + LAST
    _say(f"[large] variant={variant} env={env} T={T} H={H}")
    nbytes = kda.workspace_bytes(2, T, H, variant)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, d["cu_seqlens"],
                     d["initial_state"], variant=variant, workspace=ws if nbytes else None)
    torch.cuda.synchronize()
    if nbytes:
        off = native.error_word_offset(2)
        assert int(ws[off:off + 4].view(torch.int32).item()) == 0
    assert bool(torch.isfinite(o[:L0]).all()) and bool(torch.isfinite(fin[0]).all())
    ok, mo, mf = compare(w, o[L0:].cpu().numpy(), fin[1:].cpu().numpy(), ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    del o, fin, ws
    torch.cuda.empty_cache()
    assert ok

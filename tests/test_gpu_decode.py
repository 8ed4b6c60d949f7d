"""GPU parity of the decode step (kda_decode) against the fp64 oracle.

A decode step is the recurrence over sequences of exactly one token, so the
oracle reference is the token-loop oracle with cu_seqlens = [0, 1, ..., N].
The chained test runs a prefill (kda_fwd, split variant) and then several
decode steps on the GPU, and compares them with the oracle run over the whole
sequences in one go: the decode step must continue exactly where the prefill's
final state left off.
"""
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth
from kda_check import run_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_inputs(w, rows):
    """Device tensors [len(rows), H, 128] of the given token rows of a workload."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a[rows]).view(np.int16)).view(torch.bfloat16).cuda()

    return (bf16(w.q), bf16(w.k), bf16(w.v), torch.from_numpy(np.ascontiguousarray(w.g[rows])).cuda(),
            torch.from_numpy(np.ascontiguousarray(w.beta[rows])).cuda())


def _check(name, got, ref):
    m = synth.parity(got, ref)
    _say(f"  {name} {m}")
    assert synth.passes(m), (name, m)


def _check_bf16(name, got, ref):
    """A bf16-stored result: relative L2 gate and every element within one bf16 ulp."""
    m = synth.parity_bf16(got, ref)
    _say(f"  {name} (bf16) {m}")
    assert synth.passes_bf16(m), (name, m)


# the library picks the value-column tile per batch shape (128 columns per block for one
# token per sequence, except 64 for an fp32 state from 16,384 chains); KDA_RECURRENT_TILE
# forces each of the three block shapes
@pytest.mark.parametrize("tile", [None, "128", "64", "32"])
@pytest.mark.parametrize("N,H", [(1, 2), (7, 3), (300, 4)])
@pytest.mark.parametrize("init", [True, False])
def test_decode_step(N, H, init, tile, monkeypatch):
    import torch
    import chunked_gated_delta_kda_amd as kda

    if tile is not None:
        monkeypatch.setenv("KDA_RECURRENT_TILE", tile)
    w = synth.make_workload([1] * N, H, 100 + N, with_initial_state=init, clamp_frac=0.1)
    _say(f"[decode] N={N} H={H} init={init} tile={tile}")
    q, k, v, g, beta = _decode_inputs(w, slice(None))
    s0 = torch.from_numpy(w.initial_state).cuda() if init else None
    o, s = kda.decode(q, k, v, g, beta, w.scale, s0, state_out=torch.empty(N, H, 128, 128, device="cuda"))
    torch.cuda.synchronize()
    ro, rf = run_oracle(w)
    _check("o", o.cpu().numpy(), ro)
    _check("S", s.cpu().numpy(), rf)
    if init:   # the input state is left as it was
        np.testing.assert_array_equal(s0.cpu().numpy(), w.initial_state)


def test_decode_in_place_and_no_state_out():
    import torch
    import chunked_gated_delta_kda_amd as kda

    N, H = 33, 2
    w = synth.make_workload([1] * N, H, 7, with_initial_state=True)
    q, k, v, g, beta = _decode_inputs(w, slice(None))
    ro, rf = run_oracle(w)
    _say("[decode] state_out=None")
    o, s = kda.decode(q, k, v, g, beta, w.scale, torch.from_numpy(w.initial_state).cuda(), state_out=None)
    torch.cuda.synchronize()
    assert s is None
    _check("o", o.cpu().numpy(), ro)
    _say("[decode] in place")
    st = torch.from_numpy(w.initial_state).cuda()
    o2, s2 = kda.decode(q, k, v, g, beta, w.scale, st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    _check("o", o2.cpu().numpy(), ro)
    _check("S", s2.cpu().numpy(), rf)
    np.testing.assert_array_equal(o2.cpu().numpy(), o.cpu().numpy())


def test_prefill_then_decode():
    import torch
    import chunked_gated_delta_kda_amd as kda

    steps, H = 3, 4
    prompt = np.array([70, 1, 300, 16, 129, 0, 33])
    w = synth.make_workload(prompt + steps, H, 11, with_initial_state=True, clamp_frac=0.1)
    cu = w.cu_seqlens.astype(np.int64)
    N = w.N
    # prefill on the first len-steps tokens of every sequence
    keep = np.concatenate([np.arange(cu[n], cu[n + 1] - steps) for n in range(N)])
    pcu = np.concatenate([[0], np.cumsum(prompt)]).astype(np.int32)
    pw = synth.Workload(name="prompt", q=w.q[keep], k=w.k[keep], v=w.v[keep], g=w.g[keep],
                        beta=w.beta[keep], cu_seqlens=pcu, initial_state=w.initial_state)
    d = synth.to_device(pw)
    _say(f"[decode] prefill lengths={list(prompt)} H={H}, then {steps} decode steps")
    _, state = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                       d["initial_state"], variant="split")
    ro, rf = run_oracle(w)
    for s in range(steps):
        rows = cu[1:] - steps + s
        q, k, v, g, beta = _decode_inputs(w, rows)
        o, state = kda.decode(q, k, v, g, beta, w.scale, state)
        torch.cuda.synchronize()
        _check(f"o step {s}", o.cpu().numpy(), ro[rows])
    _check("S", state.cpu().numpy(), rf)


def _bf16_state(a):
    """bf16 device tensor of a host fp32 array (rounded to nearest even) and its exact fp32 values."""
    import torch
    bits = synth.bf16_bits(a)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return t, synth.bf16_to_f32(bits)


@pytest.mark.parametrize("N,H", [(7, 3), (300, 4)])
@pytest.mark.parametrize("tile", [None, "128", "32"])
def test_decode_bf16_state(N, H, tile, monkeypatch):
    """BF16-state form: the oracle starts from the same bf16 state values (exact in fp64)."""
    import torch
    import chunked_gated_delta_kda_amd as kda

    if tile is not None:
        monkeypatch.setenv("KDA_RECURRENT_TILE", tile)
    w = synth.make_workload([1] * N, H, 200 + N, with_initial_state=True, clamp_frac=0.1)
    s_dev, s_exact = _bf16_state(w.initial_state * np.float32(3.0))
    w.initial_state = s_exact
    _say(f"[decode] bf16 state N={N} H={H} tile={tile}")
    q, k, v, g, beta = _decode_inputs(w, slice(None))
    o, s = kda.decode(q, k, v, g, beta, w.scale, s_dev, state_out=torch.empty_like(s_dev))
    torch.cuda.synchronize()
    assert s.dtype == torch.bfloat16
    ro, rf = run_oracle(w)
    _check("o", o.cpu().numpy(), ro)
    _check_bf16("S", s.float().cpu().numpy(), rf)
    # in place gives the same bits
    o2, s2 = kda.decode(q, k, v, g, beta, w.scale, s_dev.clone())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o2.cpu().numpy(), o.cpu().numpy())
    np.testing.assert_array_equal(s2.view(torch.int16).cpu().numpy(), s.view(torch.int16).cpu().numpy())


def test_prefill_then_bf16_decode():
    """Prefill in fp32, keep the state in bf16, decode three steps; the oracle runs the
    decode steps from the same bf16-rounded prefill state."""
    import torch
    import oracle
    import chunked_gated_delta_kda_amd as kda

    steps, H = 3, 4
    prompt = np.array([70, 1, 300, 16, 129, 0, 33])
    w = synth.make_workload(prompt + steps, H, 12, with_initial_state=True, clamp_frac=0.1)
    cu = w.cu_seqlens.astype(np.int64)
    N = w.N
    keep = np.concatenate([np.arange(cu[n], cu[n + 1] - steps) for n in range(N)])
    pcu = np.concatenate([[0], np.cumsum(prompt)]).astype(np.int32)
    pw = synth.Workload(name="prompt", q=w.q[keep], k=w.k[keep], v=w.v[keep], g=w.g[keep],
                        beta=w.beta[keep], cu_seqlens=pcu, initial_state=w.initial_state)
    d = synth.to_device(pw)
    _say(f"[decode] prefill lengths={list(prompt)} H={H}, then {steps} bf16-state decode steps")
    _, state = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                       d["initial_state"], variant="split")
    state = state.to(torch.bfloat16)
    s_ref = state.float().cpu().numpy().astype(np.float64)
    for s in range(steps):
        rows = cu[1:] - steps + s
        q, k, v, g, beta = _decode_inputs(w, rows)
        # oracle: one step from the bf16 state the GPU holds
        ro, rf = oracle.kda_forward(w.q_f32()[rows], w.k_f32()[rows], w.v_f32()[rows], w.g[rows],
                                    w.beta[rows], w.scale, np.arange(N + 1), s_ref)
        o, state = kda.decode(q, k, v, g, beta, w.scale, state)
        torch.cuda.synchronize()
        _check(f"o step {s}", o.cpu().numpy(), ro)
        _check_bf16(f"S step {s}", state.float().cpu().numpy(), rf)
        s_ref = state.float().cpu().numpy().astype(np.float64)

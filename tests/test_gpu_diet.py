"""GPU parity of the input-byte diet forms of the forward: g given in bf16, and the initial
and final states held in bf16 (stored in bf16, updated in fp32: smzdm.com, "KDA 内核到底难在哪"
on the BF16 state). The oracle runs on the same values: the bf16 g and the bf16 initial state,
upcast exactly. o is held to the fp32 gate; a bf16 final state, which is at best the
rounding of the fp32 one, to the fp32 gate plus that rounding: relative L2 <= 1e-2 and
every element within one bf16 ulp (2^-7 |ref|) plus 0.02 RMS of the fp64 oracle.
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


def _diet(w, g_bf16, s_bf16):
    """The workload with g and/or the initial state rounded to bf16 (host arrays: what
    the oracle sees) and the device tensors the library receives."""
    import torch

    g = synth.bf16_to_f32(synth.bf16_bits(w.g)) if g_bf16 else w.g
    s0 = w.initial_state
    if s_bf16 and s0 is not None:
        s0 = synth.bf16_to_f32(synth.bf16_bits(s0)).reshape(s0.shape)
    w2 = synth.Workload(name=w.name, q=w.q, k=w.k, v=w.v, g=g.reshape(w.g.shape), beta=w.beta,
                        cu_seqlens=w.cu_seqlens, initial_state=s0, scale=w.scale)
    d = synth.to_device(w2)
    if g_bf16:
        d["g"] = d["g"].to(torch.bfloat16)      # exact: the values are bf16 already
    if s_bf16 and d["initial_state"] is not None:
        d["initial_state"] = d["initial_state"].to(torch.bfloat16)
    return w2, d


def _run(w, g_bf16, s_bf16, variant):
    import torch
    import chunked_gated_delta_kda_amd as kda

    w2, d = _diet(w, g_bf16, s_bf16)
    sdt = torch.bfloat16 if s_bf16 else torch.float32
    o, f = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                   d["initial_state"], variant=variant, state_dtype=sdt, check=True)
    torch.cuda.synchronize()
    assert f.dtype == sdt
    return w2, o.cpu().numpy(), f.float().cpu().numpy()


def _check(w2, o, f, s_bf16, label):
    ro, rf = run_oracle(w2)
    mo = synth.parity(o, ro)
    mf = synth.parity_bf16(f, rf, synth.GATE_MAX_ABS_RMS) if s_bf16 else synth.parity(f, rf)
    _say(f"  {label}: o {mo}\n  S {mf}")
    assert synth.passes(mo)
    assert synth.passes_bf16(mf) if s_bf16 else synth.passes(mf)


DIETS = [(True, False), (False, True), (True, True)]
SHAPES = [([300, 0, 129, 700, 17], 3, 61), ([33, 250, 0, 129], 2, 62), ([1], 2, 63)]


@pytest.mark.parametrize("variant", ["split", "recurrent"])
@pytest.mark.parametrize("diet", DIETS, ids=["g", "state", "g_state"])
@pytest.mark.parametrize("shape", SHAPES, ids=["varlen5", "varlen4", "one_token"])
def test_diet_small(shape, diet, variant):
    lengths, H, seed = shape
    g_bf16, s_bf16 = diet
    w = synth.make_workload(lengths, H, seed, with_initial_state=True, clamp_frac=0.1)
    _say(f"[diet] lengths={lengths} H={H} g_bf16={g_bf16} state_bf16={s_bf16} variant={variant}")
    w2, o, f = _run(w, g_bf16, s_bf16, variant)
    _check(w2, o, f, s_bf16, variant)


@pytest.mark.parametrize("form,segments,parts", [(401, "3", "1"), (402, "2", "1"), (401, "1", "4"),
                                                 (102, "1", "1")])
def test_diet_forms(form, segments, parts, monkeypatch):
    """Segments carry the state between launches in fp32 while the caller's states are bf16;
    the recurrence over parts composes from a bf16 initial state; a 16-token form asked for
    with bf16 inputs runs the 32-token one instead."""
    monkeypatch.setenv("KDA_RECUR_WAVES", str(form))
    monkeypatch.setenv("KDA_SEGMENTS", segments)
    monkeypatch.setenv("KDA_PARTS", parts)
    w = synth.make_workload([70, 0, 300, 16, 1, 129], 2, 64, with_initial_state=True, clamp_frac=0.1)
    _say(f"[diet] form={form} segments={segments} parts={parts}")
    w2, o, f = _run(w, True, True, "split")
    _check(w2, o, f, True, f"form {form}")


def test_diet_config3():
    """8 x 1024 tokens x 16 heads with bf16 g and bf16 states, every chain compared."""
    w = synth.config_workload(3)
    _say("[diet] config 3, bf16 g and states")
    w2, o, f = _run(w, True, True, "auto")
    _check(w2, o, f, True, "config 3")


def test_diet_config2_with_initial_state():
    """8192 tokens x 32 heads with bf16 g and bf16 initial and final states: the default
    schedule of five segments, the carry in fp32 between them and the last segment in the
    one-slice form writing the bf16 final state; every chain compared."""
    w = synth.config_workload(2)
    rng = np.random.Generator(np.random.PCG64(2002))
    s0 = (rng.standard_normal((w.N, w.H, 128, 128)) * 0.05).astype(np.float32)
    w = synth.Workload(name=w.name, q=w.q, k=w.k, v=w.v, g=w.g, beta=w.beta, cu_seqlens=w.cu_seqlens,
                       initial_state=s0, scale=w.scale)
    _say("[diet] config 2 with an initial state, bf16 g and states")
    w2, o, f = _run(w, True, True, "auto")
    _check(w2, o, f, True, "config 2")


def test_fused_rejects_diet():
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    w = synth.make_workload([40], 1, 65)
    _, d = _diet(w, True, False)
    with pytest.raises(native.KdaError):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"], variant="fused")
    torch.cuda.synchronize()

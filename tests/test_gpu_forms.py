"""GPU parity of every recurrence form and chunk-range segmentation of the split variant.

The library picks one recurrence form and segment count per shape; the
KDA_RECUR_WAVES and KDA_SEGMENTS environment overrides force each of the others
here, so that every form stays checked against the fp64 oracle on shapes that
cross segment boundaries inside sequences, hold empty sequences, and carry the
state between segments through final_state, through the workspace (no final
state requested), and in place (final_state aliasing initial_state); and the
recurrence over parts of every sequence (KDA_PARTS).
"""
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth
from kda_check import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

FORMS = [8, 9, 101, 102, 401, 402]
SEGMENTS = [1, 2, 3, 8]
LENGTHS = [70, 0, 300, 16, 1, 129]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def workload():
    w = synth.make_workload(LENGTHS, 2, 2024, with_initial_state=True, clamp_frac=0.1)
    return w, run_oracle(w)


@pytest.mark.parametrize("segments", SEGMENTS)
@pytest.mark.parametrize("form", FORMS)
def test_form_and_segments(workload, form, segments, monkeypatch):
    monkeypatch.setenv("KDA_RECUR_WAVES", str(form))
    monkeypatch.setenv("KDA_SEGMENTS", str(segments))
    w, (ro, rf) = workload
    _say(f"[forms] form={form} segments={segments} lengths={LENGTHS}")
    o, f = run_gpu(w, "split")
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


@pytest.mark.parametrize("form", [101, 401])
@pytest.mark.parametrize("parts", [2, 3, 5, 16])
def test_parts(workload, parts, form, monkeypatch):
    """The recurrence over parts of every sequence (pass 1 from zero and identity entry
    states, composition, pass 2), forced on the varlen batch, over 16-token records (101)
    and 32-token fp16 records (401): some parts of the short sequences hold no chunks, and
    the empty sequence passes its initial state through."""
    monkeypatch.setenv("KDA_PARTS", str(parts))
    monkeypatch.setenv("KDA_RECUR_WAVES", str(form))
    w, (ro, rf) = workload
    _say(f"[forms] parts={parts} form={form} lengths={LENGTHS}")
    o, f = run_gpu(w, "split")
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


@pytest.mark.parametrize("pass2", [401, 402])
@pytest.mark.parametrize("parts", [2, 5])
def test_parts_pass2_form(workload, parts, pass2, monkeypatch):
    """Pass 2 of the recurrence over parts in either 32-token form (one or two 16-column
    slices per block), whichever the part count would pick."""
    monkeypatch.setenv("KDA_PARTS", str(parts))
    monkeypatch.setenv("KDA_RECUR_WAVES", "401")
    monkeypatch.setenv("KDA_PARTS_FORM", str(pass2))
    w, (ro, rf) = workload
    _say(f"[forms] parts={parts} pass 2 form={pass2} lengths={LENGTHS}")
    o, f = run_gpu(w, "split")
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("segments,parts", [(1, 1), (4, 1), (1, 3)])
def test_no_final_state_and_in_place(workload, segments, parts, fp16, monkeypatch):
    import torch
    import chunked_gated_delta_kda_amd as kda

    form = (102 if parts == 1 else 101) + (300 if fp16 else 0)
    monkeypatch.setenv("KDA_RECUR_WAVES", str(form))
    monkeypatch.setenv("KDA_SEGMENTS", str(segments))
    monkeypatch.setenv("KDA_PARTS", str(parts))
    w, (ro, rf) = workload
    d = synth.to_device(w)
    _say(f"[forms] no final state, form={form} segments={segments} parts={parts}")
    o, fin = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                     d["initial_state"], output_final_state=False, variant="split")
    torch.cuda.synchronize()
    assert fin is None
    mo = synth.parity(o.cpu().numpy(), ro)
    _say(f"  o {mo}")
    assert synth.passes(mo)

    _say(f"[forms] in place (final_state is initial_state), segments={segments}")
    s = d["initial_state"].clone()
    o2, fin2 = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                       s, variant="split", final_state=s)
    torch.cuda.synchronize()
    assert fin2.data_ptr() == s.data_ptr()
    ok, mo, mf = compare(w, o2.cpu().numpy(), fin2.cpu().numpy(), ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok
    # deterministic: same kernels, same schedule, same result
    np.testing.assert_array_equal(o2.cpu().numpy(), o.cpu().numpy())

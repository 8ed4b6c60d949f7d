"""What the algebra fixes about the edge-case workloads, checked on the oracle (CPU)."""
import numpy as np

import oracle
from chunked_gated_delta_kda_amd import synth
from edge_cases import CASES


def test_no_write_is_a_decaying_read_out():
    """beta = 0: S_T = Diag(e^{sum of clamped g}) S_0 for every sequence."""
    w = CASES["no_write"]()
    ro, rf = oracle.kda_forward(**synth.oracle_inputs(w))
    cu = w.cu_seqlens
    for n in range(w.N):
        G = np.maximum(w.g[cu[n]:cu[n + 1]].astype(np.float64), -5.0).sum(axis=0)   # [H, 128]
        expect = np.exp(G)[:, :, None] * w.initial_state[n].astype(np.float64)
        np.testing.assert_allclose(rf[n], expect, rtol=1e-9, atol=1e-12)


def test_unit_write_returns_scaled_v():
    """beta = 1, q = k: o = scale v up to the bf16 rounding of the unit keys."""
    w = CASES["unit_write"]()
    ro, rf = oracle.kda_forward(**synth.oracle_inputs(w))
    v = w.v_f32().astype(np.float64)
    assert np.max(np.abs(ro - w.scale * v)) < 0.02 * w.scale * np.sqrt(np.mean(v * v))


def test_deep_clamp_equals_clamped_input():
    """g below -5 acts as -5: the raw and the pre-clamped inputs give identical results."""
    w = CASES["deep_clamp"]()
    a = oracle.kda_forward(**synth.oracle_inputs(w))
    inp = synth.oracle_inputs(w)
    inp["g"] = np.maximum(inp["g"], -5.0)
    b = oracle.kda_forward(**inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_slow_forget_remembers_its_entry_state():
    """After 4,096 tokens with g = 0 and beta ~ 0.05 the entry state still carries weight,
    so a composition of parts S_out = M S_in + B is exercised with M of order 1."""
    w = CASES["slow_forget"]()
    inp = synth.oracle_inputs(w)
    _, rf = oracle.kda_forward(**inp, pairs=[(0, 0)])
    _, rf0 = oracle.kda_forward(**{**inp, "initial_state": None}, pairs=[(0, 0)])
    share = np.linalg.norm(rf[0, 0] - rf0[0, 0]) / np.linalg.norm(w.initial_state[0, 0])
    assert share > 0.2, share

"""CPU tests: seeded workload generation and the parity metric."""
import numpy as np
import pytest
import torch

from chunked_gated_delta_kda_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 1e-30, 3e38], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_config_is_deterministic_and_distributed_as_stated():
    a = synth.config_workload(1)
    b = synth.config_workload(1)
    for f in ("q", "k", "v", "g", "beta", "cu_seqlens"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.q.shape == (256, 2, 128) and a.beta.shape == (256, 2)
    assert a.initial_state is None and list(a.cu_seqlens) == [0, 256]
    norms = np.linalg.norm(a.k_f32(), axis=-1)
    assert np.allclose(norms, 1.0, atol=1e-2)
    assert (a.g <= 0).all() and (a.g >= -5).all()
    assert (a.beta > 0).all() and (a.beta < 1).all()
    assert a.scale == pytest.approx(1 / np.sqrt(128), rel=1e-7)


def test_skewed_lengths():
    rng = np.random.Generator(np.random.PCG64(5))
    L = synth.skewed_lengths(rng)
    assert L.size == 12 and L.sum() == 32768 and (L >= 1).all()
    assert (L % 16 != 0).any()


def test_clamp_fraction():
    w = synth.make_workload([64], 8, 4, clamp_frac=0.1)
    at = (w.g == -5.0).all(axis=0)        # channels fixed at the clamp over time
    assert 0.03 < at.mean() < 0.2


def test_parity_metric():
    ref = np.array([1.0, -1.0, 2.0, -2.0])
    m = synth.parity(ref + np.array([0.0, 0.0, 0.0, 0.03]), ref)
    rms = np.sqrt(10 / 4)
    assert m["max_abs_rms"] == pytest.approx(0.03 / rms)
    assert m["rel_l2"] == pytest.approx(0.03 / np.sqrt(10))
    assert synth.passes(m, rel=1e-2, mx=2e-2)
    assert not synth.passes(synth.parity(ref * 1.1, ref))
    assert not synth.passes(synth.parity(np.array([np.nan, 0, 0, 0]), ref))
    z = synth.parity(np.zeros(3), np.zeros(3))
    assert synth.passes(z)


def test_bf16_result_gate():
    """The bf16 gate accepts the round-to-nearest of the reference and rejects an element
    two bf16 ulps away."""
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(4096) * np.exp(rng.uniform(-6, 3, 4096))
    rounded = synth.bf16_to_f32(synth.bf16_bits(ref.astype(np.float32))).astype(np.float64)
    m = synth.parity_bf16(rounded, ref)
    assert synth.passes_bf16(m) and m["max_err_over_bf16_bound"] <= 0.51
    # the same rounding fails the fp32 max-abs gate once large elements dominate
    bad = rounded.copy()
    i = int(np.argmax(np.abs(ref)))
    e = int(np.floor(np.log2(abs(ref[i]))))
    bad[i] += 2 * 2.0 ** (e - 7) * np.sign(ref[i])
    assert not synth.passes_bf16(synth.parity_bf16(bad, ref))

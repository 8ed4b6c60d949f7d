"""Checks that pin the fp64 oracle to facts other than itself.

Each check takes an oracle entry point ``fwd`` (same signature as
``oracle.kda_forward``) and raises AssertionError when the oracle disagrees
with a fact the recurrence fixes. test_oracle.py runs them against the real
oracle; test_oracle_mutants.py runs them against deliberately broken copies
of the oracle and expects at least one to fail for each copy.
"""
import json
import math
import os

import numpy as np

from oracle import forms

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _rand(rng, T, H, dk, dv, unit_keys=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, b


def check_golden(fwd):
    """Hand-worked tiny cases (tests/golden/hand_worked.json)."""
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        s0 = None if c["initial_state"] is None else np.array(c["initial_state"], dtype=np.float64)
        o, fin = fwd(np.array(c["q"], float), np.array(c["k"], float), np.array(c["v"], float),
                     np.array(c["g"], float), np.array(c["beta"], float), c["scale"],
                     np.array(c["cu_seqlens"]), s0)
        np.testing.assert_allclose(o, np.array(c["o"], float), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(fin, np.array(c["final_state"], float), rtol=0, atol=1e-12,
                                   err_msg=c["name"])


def check_single_token(fwd):
    """T=1 closed form: S1 = D S0 + b k (v - (D S0)^T k)^T, o = scale S1^T q."""
    rng = np.random.default_rng(11)
    dk, dv, H = 6, 4, 3
    q, k, v, g, b = _rand(rng, 1, H, dk, dv)
    g[0, 0, 1] = -9.0  # below the clamp
    s0 = rng.standard_normal((1, H, dk, dv))
    o, fin = fwd(q, k, v, g, b, 0.7, None, s0)
    for h in range(H):
        D = np.exp(np.maximum(g[0, h], -5.0))
        DS = D[:, None] * s0[0, h]
        u = b[0, h] * (v[0, h] - DS.T @ k[0, h])
        S1 = DS + np.outer(k[0, h], u)
        np.testing.assert_allclose(fin[0, h], S1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[0, h], 0.7 * S1.T @ q[0, h], rtol=0, atol=1e-12)


def check_beta_zero(fwd):
    """beta = 0: nothing is written; o_t = scale (e^{G_t} * q_t)^T S0, S_T = Diag(e^{G_T}) S0,
    with G_t the cumulative clamped log-decay since the sequence start."""
    rng = np.random.default_rng(12)
    dk, dv, H = 5, 7, 2
    lens = [9, 0, 4]
    T = sum(lens)
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    g[3, 1, :] = -6.5
    b[:] = 0.0
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((3, H, dk, dv))
    o, fin = fwd(q, k, v, g, b, 0.25, cu, s0)
    for n in range(3):
        for h in range(H):
            G = np.zeros(dk)
            for t in range(cu[n], cu[n + 1]):
                G = G + np.maximum(g[t, h], -5.0)
                np.testing.assert_allclose(o[t, h], 0.25 * (np.exp(G) * q[t, h]) @ s0[n, h],
                                           rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(fin[n, h], np.exp(G)[:, None] * s0[n, h], rtol=1e-12, atol=1e-12)


def check_orthogonal_keys_linear_attention(fwd):
    """Distinct one-hot keys and S0 = 0 make every write land on its own key row, so KDA
    becomes gated causal linear attention: o_t = scale sum_{s<=t} b_s e^{G_t[i_s]-G_s[i_s]}
    q_t[i_s] v_s. Evaluated as one masked matrix product. With g = 0 it is plain causal
    linear attention o = scale * tril(Q K^T) (b V)."""
    rng = np.random.default_rng(13)
    dk, dv, T = 24, 5, 20
    idx = rng.permutation(dk)[:T]
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    b = rng.uniform(0.1, 1.0, (T, 1))
    for zero_gate in (True, False):
        g = np.zeros((T, 1, dk)) if zero_gate else -rng.uniform(0.0, 6.0, (T, 1, dk))
        G = np.cumsum(np.maximum(g[:, 0], -5.0), axis=0)          # [T, dk]
        # decay from s to t on the key row i_s
        dec = np.exp(G[:, idx] - G[np.arange(T), idx][None, :])   # [t, s]
        M = np.tril(q[:, 0][:, idx] * dec) * b[:, 0][None, :]       # [t, s]
        ref = 0.5 * M @ v[:, 0]
        o, _ = fwd(q, k, v, g, b, 0.5, None, None)
        np.testing.assert_allclose(o[:, 0], ref, rtol=1e-12, atol=1e-12)
        if zero_gate:
            plain = 0.5 * np.tril(q[:, 0] @ k[:, 0].T) @ (b * v[:, 0])
            np.testing.assert_allclose(o[:, 0], plain, rtol=1e-12, atol=1e-12)


def check_unit_write_readback(fwd):
    """b = 1, q = k, ||k|| = 1: after the write S^T k = v exactly, so o_t = scale v_t for any
    decay and any history."""
    rng = np.random.default_rng(14)
    dk, dv, T, H = 8, 6, 30, 2
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    b[:] = 1.0
    s0 = rng.standard_normal((1, H, dk, dv))
    o, _ = fwd(k, k, v, g, b, 0.3, None, s0)
    np.testing.assert_allclose(o, 0.3 * v, rtol=1e-11, atol=1e-11)


def check_matrix_form(fwd):
    """Agreement with the explicit (I - b k k^T) Diag(e^g) S + b k v^T matrix recurrence,
    varlen with an empty sequence, dk != dv."""
    rng = np.random.default_rng(15)
    dk, dv, H = 6, 5, 2
    lens = [7, 0, 12, 1]
    T = sum(lens)
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    g[2, 0, :3] = -8.0
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((4, H, dk, dv))
    o, fin = fwd(q, k, v, g, b, 0.4, cu, s0)
    o2, fin2 = forms.matrix_form(q, k, v, g, b, 0.4, cu, s0)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin, fin2, rtol=1e-12, atol=1e-12)


def check_chunked_forms(fwd):
    """Agreement with the chunked WY rewrite for several chunk sizes and inverse methods."""
    rng = np.random.default_rng(16)
    dk, dv, H = 8, 8, 2
    lens = [37, 16, 5]
    T = sum(lens)
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((3, H, dk, dv)) * 0.1
    o, fin = fwd(q, k, v, g, b, 0.35, cu, s0)
    for C, inv, anc in ((1, "subst", False), (3, "subst", False), (16, "subst", False),
                        (16, "neumann", False), (32, "neumann", True), (64, "subst", True)):
        o2, fin2 = forms.chunked_form(q, k, v, g, b, 0.35, cu, s0, chunk=C, inverse=inv, anchor=anc)
        np.testing.assert_allclose(o, o2, rtol=1e-10, atol=1e-11, err_msg=f"C={C} {inv}")
        np.testing.assert_allclose(fin, fin2, rtol=1e-10, atol=1e-11, err_msg=f"C={C} {inv}")


def check_scalar_gate_is_gated_deltanet(fwd):
    """g constant across channels: KDA reduces to Gated DeltaNet, where the scalar decay
    commutes with the projection: S_t = a_t (I - b k k^T) S_{t-1} + b k v^T.
    With per-channel g the order matters, and the oracle must apply the decay before the
    projection (it must differ from the projection-then-decay order)."""
    rng = np.random.default_rng(17)
    dk, dv, T = 7, 4, 25
    q, k, v, g, b = _rand(rng, T, 1, dk, dv)
    gs = g[:, :, :1].repeat(dk, axis=2)
    s0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = fwd(q, k, v, gs, b, 0.6, None, s0)
    S = s0[0, 0].copy()
    ref = np.zeros((T, dv))
    for t in range(T):
        a = math.exp(max(gs[t, 0, 0], -5.0))
        kt = k[t, 0]
        S = a * (S - b[t, 0] * np.outer(kt, kt @ S)) + b[t, 0] * np.outer(kt, v[t, 0])
        ref[t] = 0.6 * S.T @ q[t, 0]
    np.testing.assert_allclose(o[:, 0], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-11, atol=1e-12)
    # per-channel: projection-then-decay is a different operator
    o_pc, _ = fwd(q, k, v, g, b, 0.6, None, s0)
    S = s0[0, 0].copy()
    wrong = np.zeros((T, dv))
    for t in range(T):
        kt = k[t, 0]
        S = np.exp(np.maximum(g[t, 0], -5.0))[:, None] * (S - b[t, 0] * np.outer(kt, kt @ S)) \
            + b[t, 0] * np.outer(kt, v[t, 0])
        wrong[t] = 0.6 * S.T @ q[t, 0]
    assert np.max(np.abs(o_pc[:, 0] - wrong)) > 1e-3


def check_g_zero_is_deltanet(fwd):
    """g = 0: no decay, and KDA is the plain delta rule (DeltaNet),
    S_t = S_{t-1} + b k (v - S_{t-1}^T k)^T, o_t = scale S_t^T q_t."""
    rng = np.random.default_rng(23)
    dk, dv, T = 6, 5, 30
    q, k, v, _, b = _rand(rng, T, 1, dk, dv)
    g = np.zeros((T, 1, dk))
    s0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = fwd(q, k, v, g, b, 0.4, None, s0)
    S = s0[0, 0].copy()
    for t in range(T):
        kt = k[t, 0]
        S = S + b[t, 0] * np.outer(kt, v[t, 0] - S.T @ kt)
        np.testing.assert_allclose(o[t, 0], 0.4 * S.T @ q[t, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-11, atol=1e-12)


def check_non_expansive(fwd):
    """With b ||k||^2 in [0, 2] and g <= 0 the step matrix (I - b k k^T) Diag(e^g) has
    spectral norm <= 1, so ||S_t||_2 <= ||S_{t-1}||_2 + b_t ||k_t|| ||v_t|| along a chain
    (checked on every prefix of one sequence, with keys of norm up to sqrt(2))."""
    rng = np.random.default_rng(29)
    dk, dv, T = 8, 6, 24
    q, k, v, g, b = _rand(rng, T, 1, dk, dv)
    k = k * rng.uniform(0.2, math.sqrt(2.0), size=(T, 1, 1))
    s0 = 3.0 * rng.standard_normal((1, 1, dk, dv))
    prev = np.linalg.norm(s0[0, 0], 2)
    for t in range(1, T + 1):
        _, fin = fwd(q[:t], k[:t], v[:t], g[:t], b[:t], 1.0, None, s0)
        cur = np.linalg.norm(fin[0, 0], 2)
        bound = prev + b[t - 1, 0] * np.linalg.norm(k[t - 1, 0]) * np.linalg.norm(v[t - 1, 0])
        assert cur <= bound + 1e-12, (t, cur, bound)
        prev = cur


def check_resume_and_packing(fwd):
    """Splitting a sequence and chaining final -> initial state, and packing sequences with
    cu_seqlens, both reproduce the single run."""
    rng = np.random.default_rng(18)
    dk, dv, H = 5, 6, 2
    T = 23
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dk, dv))
    o, fin = fwd(q, k, v, g, b, 0.5, None, s0)
    a = 9
    oa, fa = fwd(q[:a], k[:a], v[:a], g[:a], b[:a], 0.5, None, s0)
    ob, fb = fwd(q[a:], k[a:], v[a:], g[a:], b[a:], 0.5, None, fa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fb, fin, rtol=1e-12, atol=1e-12)
    # packed: [a tokens from fa-less start | rest] as two sequences equals two runs
    cu = np.array([0, a, T])
    s0p = np.concatenate([s0, fa])
    op, fp = fwd(q, k, v, g, b, 0.5, cu, s0p)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fp[1], fin[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fp[0], fa[0], rtol=1e-12, atol=1e-12)


def check_linearity_and_heads(fwd):
    """For fixed q, k, g, b the map (v, S0) -> (o, S_T) is linear; heads are independent
    (permuting heads permutes outputs)."""
    rng = np.random.default_rng(19)
    dk, dv, H, T = 6, 3, 3, 14
    q, k, v, g, b = _rand(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v.shape)
    s0, s02 = rng.standard_normal((2, 1, H, dk, dv))
    o1, f1 = fwd(q, k, v, g, b, 0.9, None, s0)
    o2, f2 = fwd(q, k, v2, g, b, 0.9, None, s02)
    o3, f3 = fwd(q, k, 2.0 * v - 3.0 * v2, g, b, 0.9, None, 2.0 * s0 - 3.0 * s02)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(f3, 2.0 * f1 - 3.0 * f2, rtol=1e-10, atol=1e-10)
    perm = np.array([2, 0, 1])
    op, fp = fwd(q[:, perm], k[:, perm], v[:, perm], g[:, perm], b[:, perm], 0.9, None, s0[:, perm])
    np.testing.assert_allclose(op, o1[:, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(fp, f1[:, perm], rtol=0, atol=1e-13)


def check_clamp(fwd):
    """Every g below -5 acts exactly as -5 (lower_bound)."""
    rng = np.random.default_rng(20)
    dk, dv, T = 4, 4, 10
    q, k, v, g, b = _rand(rng, T, 1, dk, dv)
    g_lo = g.copy()
    g_lo[::2, :, ::2] = -11.0
    g_at = g.copy()
    g_at[::2, :, ::2] = -5.0
    s0 = rng.standard_normal((1, 1, dk, dv))
    o1, f1 = fwd(q, k, v, g_lo, b, 1.0, None, s0)
    o2, f2 = fwd(q, k, v, g_at, b, 1.0, None, s0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


ALL_CHECKS = [check_golden, check_single_token, check_beta_zero,
              check_orthogonal_keys_linear_attention, check_unit_write_readback, check_matrix_form,
              check_chunked_forms, check_scalar_gate_is_gated_deltanet, check_g_zero_is_deltanet,
              check_non_expansive, check_resume_and_packing, check_linearity_and_heads, check_clamp]

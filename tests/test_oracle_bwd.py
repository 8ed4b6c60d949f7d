"""CPU pins of the backward oracle (oracle/kda_oracle_bwd.c): its gradients are checked
against things other than itself.

- Central finite differences of the forward oracle (itself pinned by test_oracle*.py) on
  tiny inputs, for every input: q, k, v, g, beta and the initial state, with a loss that
  reads both o and the final state.
- The adjoint identity: o and the final state are linear in (v, S0) jointly, so
  <do, o> + <dS_T, S_T> = <dv, v> + <dS0, S0> exactly.
- Per token, o_t is linear in q_t: <dq_t, q_t> = <do_t, o_t>.
- beta = 0 (nothing is written): closed forms of dq, dS0, dg, with dk = dv = 0.
- The clamp: below the bound g gets no gradient; at the bound the one-sided derivative from
  above is the gradient (a clamp from below passes it at equality).
Mutants of the backward oracle (one plausible mistake each) must fail one of them.
"""
import ctypes
import functools
import os
import shutil

import numpy as np
import pytest

import oracle
from oracle import build as obuild

LB = -5.0


def _inputs(rng, lengths, H, dk, dv, g_lo=-3.0):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    x = dict(q=rng.standard_normal((T, H, dk)) / np.sqrt(dk), k=rng.standard_normal((T, H, dk)) / np.sqrt(dk),
             v=rng.standard_normal((T, H, dv)), g=rng.uniform(g_lo, -0.01, (T, H, dk)),
             beta=rng.uniform(0.05, 0.95, (T, H)),
             initial_state=rng.standard_normal((len(lengths), H, dk, dv)) * 0.3)
    return x, cu


def _loss(x, cu, scale, do, dsf, lib=None):
    o, f = oracle.kda_forward(**x, scale=scale, cu_seqlens=cu, lib=lib)
    return float(np.sum(do * o) + np.sum(dsf * f))


def _grads(x, cu, scale, do, dsf, lib=None):
    return oracle.kda_backward(**x, scale=scale, d_out=do, cu_seqlens=cu, d_final_state=dsf, lib=lib)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "initial_state": "d_initial_state"}


def check_finite_differences(lib=None, fwd_lib=None):
    rng = np.random.default_rng(11)
    x, cu = _inputs(rng, [3, 0, 4], 2, 4, 3)
    scale = 0.7
    T, H = x["q"].shape[:2]
    do = rng.standard_normal((T, H, 3))
    dsf = rng.standard_normal(x["initial_state"].shape)
    gr = _grads(x, cu, scale, do, dsf, lib=lib)
    h = 1e-6
    worst = 0.0
    for name, gname in NAMES.items():
        arr = x[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(x, cu, scale, do, dsf, fwd_lib)
            arr[idx] = old - h
            lm = _loss(x, cu, scale, do, dsf, fwd_lib)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - gr[gname])) / max(1.0, np.max(np.abs(fd)))
        worst = max(worst, err)
        assert err < 1e-6, (name, err)
    return worst


def check_adjoint_identity(lib=None):
    rng = np.random.default_rng(12)
    x, cu = _inputs(rng, [40, 7, 25], 2, 128, 128)
    scale = 128 ** -0.5
    o, f = oracle.kda_forward(**x, scale=scale, cu_seqlens=cu)
    do = rng.standard_normal(o.shape)
    dsf = rng.standard_normal(f.shape)
    gr = _grads(x, cu, scale, do, dsf, lib=lib)
    lhs = np.sum(do * o) + np.sum(dsf * f)
    rhs = np.sum(gr["dv"] * x["v"]) + np.sum(gr["d_initial_state"] * x["initial_state"])
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1.0), (lhs, rhs)
    # per token: <dq_t, q_t> = <do_t, o_t>
    np.testing.assert_allclose(np.sum(gr["dq"] * x["q"], axis=-1), np.sum(do * o, axis=-1), rtol=1e-9,
                               atol=1e-12)


def check_beta_zero(lib=None):
    rng = np.random.default_rng(13)
    x, cu = _inputs(rng, [9, 14], 2, 6, 5)
    x["beta"][:] = 0.0
    x["g"][0, 0, 1] = -7.0        # one gate below the bound: acts as -5, gets no gradient
    scale = 0.4
    T, H = x["q"].shape[:2]
    do = rng.standard_normal((T, H, 5))
    dsf = rng.standard_normal(x["initial_state"].shape)
    gr = _grads(x, cu, scale, do, dsf, lib=lib)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)
    gc = np.maximum(x["g"], LB)
    for n in range(len(cu) - 1):
        for h in range(H):
            S0 = x["initial_state"][n, h]
            G = np.cumsum(gc[cu[n]:cu[n + 1], h], axis=0)          # Gamma_t, [len, dk]
            E = np.exp(G)
            qt, dot = x["q"][cu[n]:cu[n + 1], h], do[cu[n]:cu[n + 1], h]
            # o_t = scale (e^{Gamma_t} * q_t)^T S0, S_T = Diag(e^{Gamma_T}) S0
            np.testing.assert_allclose(gr["dq"][cu[n]:cu[n + 1], h], scale * E * (dot @ S0.T), rtol=1e-10,
                                       atol=1e-12)
            ds0 = scale * (E * qt).T @ dot + E[-1][:, None] * dsf[n, h]
            np.testing.assert_allclose(gr["d_initial_state"][n, h], ds0, rtol=1e-10, atol=1e-12)
            # dL/dgamma_s = sum_{t >= s} scale q_t e^{Gamma_t} (S0 do_t) + e^{Gamma_T} (S0 . dS_T) rows
            per_t = scale * qt * E * (dot @ S0.T)                   # [len, dk]
            tail = np.cumsum(per_t[::-1], axis=0)[::-1]
            dgam = tail + (E[-1] * np.sum(S0 * dsf[n, h], axis=1))[None, :]
            dgam = np.where(x["g"][cu[n]:cu[n + 1], h] >= LB, dgam, 0.0)
            np.testing.assert_allclose(gr["dg"][cu[n]:cu[n + 1], h], dgam, rtol=1e-9, atol=1e-12)
    assert gr["dg"][0, 0, 1] == 0.0


def check_clamp_boundary(lib=None):
    rng = np.random.default_rng(14)
    x, cu = _inputs(rng, [6], 1, 4, 4)
    x["g"][2, 0, 3] = LB                     # exactly at the bound
    scale = 0.6
    do = rng.standard_normal((6, 1, 4))
    dsf = rng.standard_normal(x["initial_state"].shape)
    gr = _grads(x, cu, scale, do, dsf, lib=lib)
    h = 1e-6
    l0 = _loss(x, cu, scale, do, dsf)
    x["g"][2, 0, 3] = LB + h
    lp = _loss(x, cu, scale, do, dsf)
    right = (lp - l0) / h
    assert abs(gr["dg"][2, 0, 3] - right) < 1e-5 * max(1.0, abs(right)), (gr["dg"][2, 0, 3], right)
    assert abs(right) > 1e-4      # the case is not trivially zero


ALL_CHECKS = [check_finite_differences, check_adjoint_identity, check_beta_zero, check_clamp_boundary]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_backward_oracle_pins(check):
    check()


# ---------------------------------------------------------------- mutants of the backward oracle
MUTANTS = {
    "no_dS1_term": ("for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += kt[i] * u[j];",
                    "for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += 0.0 * kt[i] * u[j];"),
    "du_sign": ("u[j] = -bt * dd[j];", "u[j] = bt * dd[j];"),
    "no_decay_of_dS": ("for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] *= a[i];",
                       "for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] *= 1.0;"),
    "dg_no_clamp_mask": ("dgt[i] = gt[i] >= J->lower_bound ? acc : 0.0;", "dgt[i] = acc;"),
    "no_dk_through_u": ("            dkt[i] += acc;", "            dkt[i] += 0.0 * acc;"),
    "dbeta_with_v": ("db += dd[j] * r[j];", "db += dd[j] * vt[j];"),
    "dq_from_S1": ("for (int64_t j = 0; j < dv; ++j) acc += S[i * dv + j] * dot[j];",
                   "for (int64_t j = 0; j < dv; ++j) acc += S1[i * dv + j] * dot[j];"),
    "half_output_gradient": ("dS[i * dv + j] += J->scale * qt[i] * dot[j];",
                                     "dS[i * dv + j] += 0.5 * J->scale * qt[i] * dot[j];"),
}


@functools.lru_cache(maxsize=None)
def _mutant_lib(name, tmpdir):
    src = open(obuild.SRC_BWD).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutant anchor not unique: {old!r}"
    path = os.path.join(tmpdir, f"mutb_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.compile_oracle([obuild.SRC, path], os.path.join(tmpdir, f"libmutb_{name}.so"), strict=False)
    return oracle._bind(ctypes.CDLL(lib))


@pytest.fixture(scope="module")
def tmpdir_mod(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants_bwd")
    yield str(d)
    shutil.rmtree(str(d), ignore_errors=True)


@pytest.mark.skipif(shutil.which(os.environ.get("CC", "gcc")) is None, reason="no C compiler")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, tmpdir_mod):
    lib = _mutant_lib(name, tmpdir_mod)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(lib=lib)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"

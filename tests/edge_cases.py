"""Edge-case workloads of the method (shared by the GPU parity tests and the CPU checks of
what the oracle gives on them).

- deep_clamp: g far below the bound on 30% of the channels (down to -1e4), which must act
  as -5 (smzdm.com, "KDA 内核到底难在哪": lower_bound = -5).
- slow_forget: g = 0 with beta ~ 0.05, a slowly forgetting chain whose entry state still
  matters after thousands of tokens (each part's linear map M is of order 1).
- no_write: beta = 0, nothing is written; o reads out the decaying initial state.
- unit_write: beta = 1 with q = k of unit norm: every write makes S^T k = v, so o = scale v.
"""
import numpy as np

from chunked_gated_delta_kda_amd import synth

LENGTHS = [700, 3, 1200, 0, 129]


def _with(w, **kw):
    d = dict(name=w.name, q=w.q, k=w.k, v=w.v, g=w.g, beta=w.beta, cu_seqlens=w.cu_seqlens,
             initial_state=w.initial_state, scale=w.scale)
    d.update(kw)
    return synth.Workload(**d)


def _deep_clamp():
    w = synth.make_workload(LENGTHS, 2, 301, with_initial_state=True)
    rng = np.random.Generator(np.random.PCG64(3010))
    g = w.g.copy()
    mask = rng.random((w.H, 128)) < 0.3                      # 30% of channels, fixed over time
    deep = -np.exp(rng.uniform(np.log(5.0), np.log(1e4), size=(w.T, w.H, 128))).astype(np.float32)
    g[:, mask] = deep[:, mask]
    assert g.min() < -1000 and (g[:, ~mask] >= -5).all()
    return _with(w, g=g, name="g down to -1e4")


def _slow_forget():
    w = synth.make_workload([4096, 300], 2, 302, with_initial_state=True)
    rng = np.random.Generator(np.random.PCG64(3020))
    beta = rng.uniform(0.03, 0.07, size=w.beta.shape).astype(np.float32)
    return _with(w, g=np.zeros_like(w.g), beta=beta, name="g = 0, beta ~ 0.05")


def _no_write():
    w = synth.make_workload(LENGTHS, 2, 303, with_initial_state=True)
    return _with(w, beta=np.zeros_like(w.beta), name="beta = 0")


def _unit_write():
    w = synth.make_workload(LENGTHS, 2, 304, with_initial_state=True)
    return _with(w, q=w.k.copy(), beta=np.ones_like(w.beta), name="beta = 1, q = k")


CASES = {"deep_clamp": _deep_clamp, "slow_forget": _slow_forget, "no_write": _no_write,
         "unit_write": _unit_write}

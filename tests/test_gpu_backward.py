"""GPU parity of the backward (kda_bwd) against the fp64 backward oracle (itself pinned by
finite differences, the adjoint identity and closed forms in test_oracle_bwd.py).

The library computes in fp32 over a token loop; every gradient is held to the forward's
fp32 gate (relative L2 <= 1e-2, max abs error <= 2e-2 RMS of the reference). Inputs: the
seeded synthetic workloads of the forward tests (bf16 q, k, v upcast exactly; fp32 g and
beta), with gates at exactly -5 (clamped channels) and some below it, ragged and empty
sequences, with and without initial state and final-state gradient.
"""
import sys

import numpy as np
import pytest

import oracle
from chunked_gated_delta_kda_amd import synth

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _grads_in(w, seed, with_dsf):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    do = rng.standard_normal((w.T, w.H, 128)).astype(np.float32)
    dsf = rng.standard_normal((w.N, w.H, 128, 128)).astype(np.float32) * np.float32(0.1) if with_dsf else None
    return do, dsf


def _below_bound(w, seed, frac=0.02):
    """Set a few gates below the bound (they act as -5 and get no gradient)."""
    rng = np.random.Generator(np.random.PCG64(2000 + seed))
    m = rng.random(w.g.shape) < frac
    w.g[m] = np.float32(-7.0)


def _run_gpu(w, do, dsf, use_cu=True):
    import torch
    import chunked_gated_delta_kda_amd as kda

    d = synth.to_device(w)
    gr = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], torch.from_numpy(do).cuda(), d["scale"],
                 d["cu_seqlens"] if use_cu else None, d["initial_state"],
                 None if dsf is None else torch.from_numpy(dsf).cuda())
    torch.cuda.synchronize()
    return {n: gr[n].cpu().numpy() for n in NAMES}


def _run_oracle(w, do, dsf):
    x = synth.oracle_inputs(w)
    return oracle.kda_backward(**x, d_out=do, d_final_state=dsf)


def _check(got, ref, label):
    ok = True
    for n in NAMES:
        m = synth.parity(got[n], ref[n])
        _say(f"  {label} {n}: rel_l2 {m['rel_l2']:.2e} max_abs/rms {m['max_abs_rms']:.2e} rms {m['rms']:.3e}")
        ok &= synth.passes(m)
    assert ok


CASES = [
    ("varlen5_init_dsf", [70, 0, 33, 1, 129], 2, 71, True, True),
    ("varlen4_no_init", [32, 64, 0, 95], 3, 72, False, True),
    ("no_dsf", [200, 17], 2, 73, True, False),
]


@pytest.mark.parametrize("name,lengths,H,seed,init,with_dsf", CASES, ids=[c[0] for c in CASES])
def test_bwd_small(name, lengths, H, seed, init, with_dsf):
    w = synth.make_workload(lengths, H, seed, with_initial_state=init, clamp_frac=0.1)
    _below_bound(w, seed)
    do, dsf = _grads_in(w, seed, with_dsf)
    _say(f"[bwd] {name} lengths={lengths} H={H}")
    got = _run_gpu(w, do, dsf)
    _check(got, _run_oracle(w, do, dsf), name)
    # below the bound: exactly no gradient
    assert np.all(got["dg"][w.g < -5.0] == 0.0)


@pytest.mark.parametrize("waves", [8, 4])
@pytest.mark.parametrize("name,lengths,H,seed,init,with_dsf", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_bwd_small_forms(monkeypatch, waves, name, lengths, H, seed, init, with_dsf):
    """Both forms on every case shape: two workgroups per chain adding onto zero (8 waves),
    four adding partial sums through a last kernel (4 waves); KDA_BWD_WAVES forces them."""
    monkeypatch.setenv("KDA_BWD_WAVES", str(waves))
    w = synth.make_workload(lengths, H, seed, with_initial_state=init, clamp_frac=0.1)
    _below_bound(w, seed)
    do, dsf = _grads_in(w, seed, with_dsf)
    _say(f"[bwd] {name}, {waves} waves per workgroup")
    got = _run_gpu(w, do, dsf)
    _check(got, _run_oracle(w, do, dsf), f"{name} w{waves}")
    assert np.all(got["dg"][w.g < -5.0] == 0.0)


def test_bwd_single_sequence_without_offsets():
    w = synth.config_workload(1)
    do, dsf = _grads_in(w, 1, True)
    _say("[bwd] 256 tokens x 2 heads, cu_seqlens NULL")
    _check(_run_gpu(w, do, dsf, use_cu=False), _run_oracle(w, do, dsf), "tiny")


def test_bwd_no_tokens():
    """T = 0: the gradient of the initial state is the final-state gradient itself."""
    w = synth.make_workload([0, 0], 2, 74, with_initial_state=True)
    do, dsf = _grads_in(w, 74, True)
    got = _run_gpu(w, do, dsf)
    assert np.array_equal(got["d_initial_state"], dsf)


def _sub_workload(w, seqs, heads):
    """The chains (sequence n, head h) for n in seqs, h in heads, as a workload of their own:
    chains are independent, so its gradients are those of the full batch's chains."""
    rows = np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs])
    lengths = [int(w.cu_seqlens[n + 1] - w.cu_seqlens[n]) for n in seqs]
    cu = np.zeros(len(seqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    hs = np.asarray(heads)
    s0 = None if w.initial_state is None else np.ascontiguousarray(w.initial_state[np.ix_(seqs, hs)])
    return synth.Workload(name=w.name + " (chains)", q=np.ascontiguousarray(w.q[rows][:, hs]),
                          k=np.ascontiguousarray(w.k[rows][:, hs]), v=np.ascontiguousarray(w.v[rows][:, hs]),
                          g=np.ascontiguousarray(w.g[rows][:, hs]), beta=np.ascontiguousarray(w.beta[rows][:, hs]),
                          cu_seqlens=cu, initial_state=s0, scale=w.scale), rows


@pytest.mark.parametrize("cfg", [3, 2])
def test_bwd_config_every_chain(cfg):
    """The full workloads, 8 x 1024 tokens x 16 heads with initial states (config 3) and
    8192 tokens x 32 heads (config 2), run whole on the GPU: every chain compared with the
    oracle, element by element."""
    w = synth.config_workload(cfg)
    _below_bound(w, cfg, frac=0.01)
    do, dsf = _grads_in(w, cfg, True)
    _say(f"[bwd] config {cfg} ({w.N} sequences, {w.T} tokens, {w.H} heads), every chain")
    _check(_run_gpu(w, do, dsf), _run_oracle(w, do, dsf), f"config {cfg}")


def test_bwd_chains_alone_match_the_batch(monkeypatch):
    """Chains are independent: two sequences x three heads of config 3 run as a batch of their
    own give the same gradients as inside the whole batch (bit for bit, with the same form:
    the forms add the column parts in different orders)."""
    monkeypatch.setenv("KDA_BWD_WAVES", "8")
    w = synth.config_workload(3)
    _below_bound(w, 3, frac=0.01)
    do, dsf = _grads_in(w, 3, True)
    got = _run_gpu(w, do, dsf)
    seqs, heads = [0, 5], [0, 7, 15]
    sw, rows = _sub_workload(w, seqs, heads)
    alone = _run_gpu(sw, np.ascontiguousarray(do[rows][:, heads]), np.ascontiguousarray(dsf[np.ix_(seqs, heads)]))
    for n in NAMES:
        sub = got[n][np.ix_(seqs, heads)] if n == "d_initial_state" else got[n][rows][:, heads]
        assert np.array_equal(sub, alone[n]), n


@pytest.mark.parametrize("waves", [8, 4])
def test_bwd_deterministic(monkeypatch, waves):
    """dq, dk, dg and dbeta are sums of two column halves added onto zero (8 waves), or of 4
    partial sums added in a fixed order (4 waves): two calls on the same inputs give the
    same bits. The forms differ only in the order of those sums."""
    monkeypatch.setenv("KDA_BWD_WAVES", str(waves))
    w = synth.make_workload([300, 77], 3, 75, with_initial_state=True, clamp_frac=0.1)
    do, dsf = _grads_in(w, 75, True)
    a = _run_gpu(w, do, dsf)
    b = _run_gpu(w, do, dsf)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n
    _check(a, _run_oracle(w, do, dsf), f"w{waves}")


@pytest.mark.parametrize("waves", [8, 4])
@pytest.mark.parametrize("parts", [2, 3, 16])
def test_bwd_parts(monkeypatch, waves, parts):
    """The backward over parts of each sequence (KDA_BWD_PARTS forces it): state maps of
    every part from zero and identity entries, composed forwards (entry states) and
    backwards (exit gradients, d_initial_state), then every part's backward. Ragged lengths,
    an empty sequence, parts with no tokens (16 parts of 5 tokens), initial state and
    final-state gradient."""
    monkeypatch.setenv("KDA_BWD_WAVES", str(waves))
    monkeypatch.setenv("KDA_BWD_PARTS", str(parts))
    w = synth.make_workload([300, 0, 77, 5], 2, 81, with_initial_state=True, clamp_frac=0.1)
    _below_bound(w, 81)
    do, dsf = _grads_in(w, 81, True)
    _say(f"[bwd] parts={parts} waves={waves}")
    _check(_run_gpu(w, do, dsf), _run_oracle(w, do, dsf), f"parts {parts} w{waves}")


def test_bwd_parts_slow_decay(monkeypatch):
    """Parts where the maps are far from zero: g = 0 (no decay) and small beta, so that a
    part's state and gradient maps stay O(1) over its 256 tokens and the composition
    carries real information from part to part."""
    monkeypatch.setenv("KDA_BWD_PARTS", "4")
    w = synth.make_workload([1024, 700], 2, 82, with_initial_state=True)
    w.g[:] = np.float32(0.0)
    w.beta[:] = np.float32(0.05)
    do, dsf = _grads_in(w, 82, True)
    _say("[bwd] parts=4, g = 0, beta = 0.05")
    _check(_run_gpu(w, do, dsf), _run_oracle(w, do, dsf), "parts slow decay")


@pytest.mark.parametrize("waves", [8, 4])
def test_bwd_parts_by_length(monkeypatch, waves):
    """Parts in proportion to each sequence's length (one per 128 tokens here, at most 8):
    700 tokens in 6 parts, 300 in 3, the short and the empty sequences in one (no state
    passes for them), the other slots empty."""
    monkeypatch.setenv("KDA_BWD_WAVES", str(waves))
    monkeypatch.setenv("KDA_BWD_PARTS", "8")
    monkeypatch.setenv("KDA_BWD_PART_TOKENS", "128")
    w = synth.make_workload([700, 40, 0, 300, 5], 2, 83, with_initial_state=True, clamp_frac=0.1)
    _below_bound(w, 83)
    do, dsf = _grads_in(w, 83, True)
    _say(f"[bwd] parts by length, waves={waves}")
    _check(_run_gpu(w, do, dsf), _run_oracle(w, do, dsf), f"parts by length w{waves}")

"""GPU parity: the HIP path against the fp64 oracle on the same bf16-rounded inputs.

Gate (on o and on final_state separately): relative L2 error <= 1e-2 and
max-abs error <= 2e-2 * RMS of the oracle's values.
"""
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth
from kda_check import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

VARIANTS = ["split", "fused", "recurrent"]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny_config_full(variant):
    w = synth.config_workload(1)
    _say(f"[parity] tiny config variant={variant}")
    o, f = run_gpu(w, variant)
    ro, rf = run_oracle(w)
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


SMALL_CASES = [
    # (lengths, H, initial_state, clamp_frac, seed)
    ([1], 1, False, 0.0, 100),
    ([17], 1, True, 0.0, 101),
    ([16, 16], 2, True, 0.0, 102),
    ([300], 3, False, 0.1, 103),
    ([5, 0, 37, 64, 1], 2, True, 0.0, 104),
    ([0], 2, True, 0.0, 105),
    ([33, 250, 0, 129], 3, False, 0.2, 106),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"L{c[0]}_H{c[1]}")
def test_small_shapes(case, variant):
    lengths, H, init, clamp, seed = case
    _say(f"[parity] small lengths={lengths} H={H} init={init} clamp={clamp} variant={variant}")
    w = synth.make_workload(lengths, H, seed, with_initial_state=init, clamp_frac=clamp)
    o, f = run_gpu(w, variant)
    ro, rf = run_oracle(w)
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    if w.T == 0:
        expect = np.zeros_like(rf) if w.initial_state is None else w.initial_state
        np.testing.assert_array_equal(f, expect)
    assert ok


@pytest.mark.parametrize("variant", VARIANTS)
def test_random_small_shapes(variant):
    rng = np.random.default_rng(7)
    for it in range(6):
        N = int(rng.integers(1, 6))
        lengths = rng.integers(0, 120, size=N)
        lengths[rng.integers(0, N)] = int(rng.integers(1, 300))
        H = int(rng.integers(1, 4))
        init = bool(rng.integers(0, 2))
        _say(f"[parity] random it={it} lengths={list(lengths)} H={H} init={init}")
        w = synth.make_workload(lengths, H, 1000 + it, with_initial_state=init, clamp_frac=0.1)
        o, f = run_gpu(w, variant)
        ro, rf = run_oracle(w)
        ok, mo, mf = compare(w, o, f, ro, rf)
        _say(f"  o {mo}\n  S {mf}")
        assert ok


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_config_all_chains(cfg):
    """The full-size workloads through the path the library picks, every output element
    and every final state compared with the oracle (which runs the whole workload)."""
    _say(f"[parity] config {cfg} ({synth.CONFIGS[cfg]['name']}) default path: generating")
    w = synth.config_workload(cfg)
    _say(f"  running GPU; lengths={list(w.lengths)[:12]}")
    o, f = run_gpu(w, "auto")
    _say("  running oracle on every chain")
    ro, rf = run_oracle(w)
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


# The other variants at full size, on sampled (sequence, head) chains that the oracle
# computes one by one; every other element is checked to be finite.
SAMPLES = {
    2: [(0, 0), (0, 13), (0, 31)],
    3: [(0, 0), (3, 7), (7, 15)],
    4: [(0, 2), (0, 5)],
    5: None,   # chosen below: longest, shortest and a middle sequence
}


@pytest.mark.parametrize("variant", ["fused", "recurrent"])
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_config_sampled(cfg, variant):
    _say(f"[parity] config {cfg} ({synth.CONFIGS[cfg]['name']}) variant={variant}: generating")
    w = synth.config_workload(cfg)
    pairs = SAMPLES[cfg]
    if pairs is None:
        L = w.lengths
        pairs = [(int(np.argmax(L)), 5), (int(np.argmin(L)), 30), (len(L) // 2, 17)]
    _say(f"  running GPU; lengths={list(w.lengths)[:12]} pairs={pairs}")
    o, f = run_gpu(w, variant)
    assert np.isfinite(o).all() and np.isfinite(f).all()
    _say("  running oracle")
    ro, rf = run_oracle(w, pairs=pairs)
    ok, mo, mf = compare(w, o, f, ro, rf, pairs=pairs)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("N,maxlen", [(700, 40), (2100, 8)])
def test_many_sequences(N, maxlen, variant):
    """More sequences than the chunk map's 256 threads (its scans carry across passes),
    and past 2048 sequences (no longest-first ranking); with 2 heads the split variant
    runs the per-chain hybrid over 1,400 and 4,200 chains. Every chain is compared."""
    rng = np.random.Generator(np.random.PCG64(N))
    lengths = rng.integers(0, maxlen + 1, size=N)
    w = synth.make_workload(lengths, 2, N, with_initial_state=True, clamp_frac=0.1)
    _say(f"[parity] many sequences N={N} T={w.T} variant={variant}")
    o, f = run_gpu(w, variant)
    ro, rf = run_oracle(w)
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok


@pytest.mark.parametrize("N", [63, 64])
def test_chunk_map_boundary(N):
    """Up to 63 sequences (32-token forms) the first prep launch forms the chunk map, one
    wave holding the offsets; from 64 a chunk-map launch does. Both sides of the boundary,
    with empty and one-token sequences, every chain compared."""
    from chunked_gated_delta_kda_amd import native
    rng = np.random.Generator(np.random.PCG64(6300 + N))
    lengths = rng.integers(2, 90, size=N)
    lengths[::9] = 0
    lengths[1::13] = 1
    w = synth.make_workload(lengths, 1, 6300 + N, with_initial_state=True, clamp_frac=0.1)
    plan = [p[0] for p in native.launch_plan(N, w.T, 1, "split")]
    assert plan[-1] == "recur" and (plan[0] == "chunk_map") == (N > 63), plan
    _say(f"[parity] chunk map boundary N={N} T={w.T} plan={plan}")
    o, f = run_gpu(w, "split")
    ro, rf = run_oracle(w)
    ok, mo, mf = compare(w, o, f, ro, rf)
    _say(f"  o {mo}\n  S {mf}")
    assert ok

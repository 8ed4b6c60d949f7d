"""HIP graph capture of the library's calls (torch.cuda.graph).

Decode loops and short prefills are launch-bound, so callers capture them. Each
case captures one call, then replays the graph three times with the program's own
eager work (other library calls, copies) and synchronisations between replays, and
checks every replay bit for bit against an eager call on the same inputs.
"""
import sys

import numpy as np
import pytest

from chunked_gated_delta_kda_amd import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _eager_noise(kda, torch):
    """Unrelated eager work between replays: a library call on other data and a copy."""
    w = synth.make_workload([40, 3], 2, 99)
    d = synth.to_device(w)
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"], None, variant="split")
    x = torch.randn(1 << 20, device="cuda")
    x.mul_(2.0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant,lengths,H", [("split", [70, 0, 300, 16, 1, 129], 2),
                                               ("split", [1024], 32),      # segmented chunk range
                                               ("recurrent", [5, 1, 12], 4)])
def test_prefill_graph_replays(variant, lengths, H):
    import torch
    import chunked_gated_delta_kda_amd as kda

    w = synth.make_workload(lengths, H, 31, with_initial_state=True, clamp_frac=0.1)
    d = synth.to_device(w)
    nws = kda.workspace_bytes(w.N, w.T, w.H, variant)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(w.T, w.H, 128, device="cuda")
    fin = torch.empty(w.N, w.H, 128, 128, device="cuda")

    def call():
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"], d["initial_state"],
                variant=variant, out=out, final_state=fin, workspace=ws)

    _say(f"[graph] prefill variant={variant} lengths={lengths} H={H}")
    call()                                   # eager: reference, and kernel attributes set
    torch.cuda.synchronize()
    ref_o, ref_f = out.cpu().numpy().copy(), fin.cpu().numpy().copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        out.zero_()
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref_o, err_msg=f"replay {rep}: o")
        np.testing.assert_array_equal(fin.cpu().numpy(), ref_f, err_msg=f"replay {rep}: final state")
        _eager_noise(kda, torch)


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_decode_graph_replays(state_dtype):
    import torch
    import chunked_gated_delta_kda_amd as kda

    N, H = 96, 8
    w = synth.make_workload([1] * N, H, 32, with_initial_state=True)
    d = synth.to_device(w)
    s_init = d["initial_state"] if state_dtype == "f32" else d["initial_state"].to(torch.bfloat16)
    state = s_init.clone()
    out = torch.empty(N, H, 128, device="cuda")

    def call():
        kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, state, out=out)

    _say(f"[graph] decode N={N} H={H} state={state_dtype}")
    call()
    torch.cuda.synchronize()
    ref_o, ref_s = out.cpu().numpy().copy(), state.float().cpu().numpy().copy()
    state.copy_(s_init)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        state.copy_(s_init)                  # each replay steps from the same state
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref_o, err_msg=f"replay {rep}: o")
        np.testing.assert_array_equal(state.float().cpu().numpy(), ref_s, err_msg=f"replay {rep}: state")
        _eager_noise(kda, torch)

"""Helpers shared by the GPU tests: run the HIP path and the oracle on one workload."""
import numpy as np

import oracle
from chunked_gated_delta_kda_amd import synth


def run_gpu(w, variant="auto", **kw):
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    d = synth.to_device(w)
    nbytes = kda.workspace_bytes(w.N, w.T, w.H, variant)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                     d["initial_state"], variant=variant, workspace=ws, **kw)
    torch.cuda.synchronize()
    if nbytes:   # variants with a workspace hold a device error word in it
        off = native.error_word_offset(w.N)
        err = int(ws[off:off + 4].view(torch.int32).item())
        assert err == 0, f"device error word set ({err})"
    return o.cpu().numpy(), fin.cpu().numpy()


def run_oracle(w, pairs=None):
    return oracle.kda_forward(**synth.oracle_inputs(w), pairs=pairs)


def rows_of(w, pairs):
    """Boolean mask [T, H] of the output rows owned by the given (sequence, head) chains."""
    m = np.zeros((w.T, w.H), dtype=bool)
    for n, h in pairs:
        m[w.cu_seqlens[n]:w.cu_seqlens[n + 1], h] = True
    return m


def compare(w, got_o, got_f, ref_o, ref_f, pairs=None, rel=synth.GATE_REL_L2, mx=synth.GATE_MAX_ABS_RMS):
    """Parity metrics over all outputs, or over the chains in ``pairs`` only."""
    if pairs is None:
        mo = synth.parity(got_o, ref_o)
        mf = synth.parity(got_f, ref_f)
    else:
        rows = rows_of(w, pairs)
        mo = synth.parity(got_o[rows], ref_o[rows])
        idx = tuple(np.array(pairs).T)
        mf = synth.parity(got_f[idx], ref_f[idx])
    ok = synth.passes(mo, rel, mx) and synth.passes(mf, rel, mx)
    return ok, mo, mf

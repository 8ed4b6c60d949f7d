#!/usr/bin/env python3
"""KDA forward (prefill) benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--variant auto]
    python bench.py --decode 256 [--heads 32]     # decode step (kda_decode) instead

A step is one kda_fwd call over the whole synthetic workload (chunk map,
chunk prep and the sequential recurrence: every kernel of the path) with the
inputs already resident in device memory. W untimed steps, then exactly K
timed steps bracketed by device synchronisation. Prints one JSON line.

Per-kernel durations come from HIP events that the library records on its
stream before its first kernel launch and after each launch
(kda_options.stage_events), in every EVENT_EVERY-th of the timed steps (each
record costs about a microsecond of device time); kda_launch_plan names the
launches. When the recurrence leaves CUs idle, the split variant cuts the chunk
range into segments and prepares segment s+1 inside the launch that runs the
recurrence of segment s: then a kernel kind has several launches per step, and
its time is their sum. The CPU baseline is the fp64 oracle on the host cores, timed in
the same run on the same inputs; it also provides the parity check printed
with the result.

After the timed steps, COLD_STEPS more steps run each after a 512 MiB device write that
evicts the L2s and the last-level cache; their median (HIP events around the call) is
reported as "cold".

With --decode N a step is one kda_decode call: one token for each of N sequences,
the fp32 state updated in place, as in a decode loop; that mode prints its own
JSON line (decode tokens/s, roofline against HBM for the state traffic).

With --backward a step is one kda_bwd call (all gradients) over the --config workload;
that mode prints its own JSON line (backward tokens/s), with parity of sampled chains
against the backward oracle.
"""
import argparse
import contextlib
import ctypes
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from chunked_gated_delta_kda_amd import synth  # noqa: E402


@contextlib.contextmanager
def no_gc():
    """No garbage-collector pause inside a timed region (collect before it)."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()

METRIC = "KDA prefill fwd tokens/s + % bf16 MFMA peak, 1 MI355X (T=8192, dk=dv=128)"
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FLOP_PER_TOKEN_HEAD = 121856      # chunked method at C=16: 6 d^2 + 2C(3d + 2d) + 12 C^2, d = 128
STATE_BYTES = 128 * 128 * 4       # one (sequence, head) state, fp32
# Algorithmic bytes of the path per token-head (the unit): q, k, v bf16 (3 x 256) + g fp32
# (512) + beta fp32 (4) + o fp32 (512) = 1796 B; with bf16 g, 1540 B. Plus 64 KiB per
# (sequence, head) for each state read or written (32 KiB in bf16). A launch is credited
# with the unit's bytes for every token-head it processes (the roofline's "achieved");
# the bytes its own inputs and outputs amount to are reported beside ("own_bytes").
BYTES_PER_TOKEN_HEAD = 1796
KERNEL_OWN_BYTES_PER_TOKEN_HEAD = {"prep": 2 * 256 + 512 + 4, "recur": 256 + 512}
GATED_CONFIG = 3                  # the T=8192 varlen prefill the target sentence names
GATED_BAR_US = 52.5               # 60% of the HBM roofline for its 252.2 MB
OTHER_CONFIGS = (1, 4, 5)         # timed after the headline line's two, unless --no-others
DECODE_METRIC = "KDA decode step tokens/s, 1 MI355X (one token per sequence, dk=dv=128)"
EVENT_EVERY = 4                   # timed steps per step that records kernel events
COLD_STEPS = 20                   # extra steps timed after a cache-evicting device write each
COLD_FLUSH_BYTES = 512 << 20      # > the 256 MB last-level cache (MALL) plus the L2s
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded (libkda.so binds to the same one)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def array(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            # timing-only events: no system-scope fence (cache writeback) at each record;
            # they are read after a full device synchronisation
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            arr[i] = e.value
            self.made.append(e.value)
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


# the sources each kernel kind is built and launched from
_COMMON_SOURCES = ("kda_api.cpp", "kda_launch.hpp")
KIND_SOURCES = {"recurrent": _COMMON_SOURCES + ("kda_recurrent.hip",),
                "fused": _COMMON_SOURCES + ("kda_device.hpp", "kda_fused.hip")}
_CHUNKED_SOURCES = _COMMON_SOURCES + ("kda_device.hpp", "kda_split.hip", "kda_h32.hip")


def _code_only(text):
    """C++ source without comments and blank-line/indent differences: a comment edit
    leaves the kernels, and so the hash, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                       # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(" ".join(line.split()) for line in "".join(out).splitlines() if line.strip())


def kernel_source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_gated_delta_kda_amd", "csrc")
    for f in sorted(KIND_SOURCES.get(kind, _CHUNKED_SOURCES)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("kernels", {}).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel) or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def ingest_pmc(fetch_csv, write_csv, workload, command):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    profiles/traffic.json. Each counter is scaled by the ratio of true bytes to counted
    bytes for the plain device copy that --copy-calibration runs in the same process
    (the largest copy dispatch moves the same known number of bytes each way)."""
    import collections
    import csv
    import re

    def load(path, counter):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                per[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no copy kernel in the counter run (use --copy-calibration)")
    true_bytes = max(max(fetch[copy[0]]), max(write[copy[0]]))   # read == written for a copy
    f_scale = true_bytes / max(fetch[copy[0]])
    w_scale = true_bytes / max(write[copy[0]])
    out = {"workload": workload, "command": command, "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration_bytes": true_bytes, "kernels": {}}
    kinds = collections.defaultdict(lambda: ([], []))
    for name in fetch:
        m = re.search(r"kda::(?:\(anonymous namespace\)::)?(\w+?)_kernel", name)
        if not m or name not in write:
            continue
        base = m.group(1)      # e.g. prep, recur_pair, recur_prep, fused, chunk_map
        kind = ("recurrent" if base in ("recurrent", "decode") else
                "parts" if base.startswith("parts") or base.endswith("_parts") else
                "recur_prep" if base.startswith("recur") and base.endswith("_prep") else
                "recur" if base.startswith("recur") else
                "prep" if base.startswith("prep") else base)
        kinds[kind][0].extend(fetch[name])
        kinds[kind][1].extend(write[name])
    for kind, (fl, wl) in kinds.items():
        # mean over dispatches: segment launches of one kind cover different chunk ranges
        fb = float(np.mean(fl)) * f_scale
        wb = float(np.mean(wl)) * w_scale
        out["kernels"][f"{kind}@{workload}"] = {"workload": workload, "source_hash": kernel_source_hash(kind),
                                "command": command, "fetch_scale": f_scale, "write_scale": w_scale,
                                "fetch_bytes": fb, "write_bytes": wb, "dispatches": len(fl),
                                "bytes_per_launch": fb + wb}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    prev = {}
    if os.path.exists(TRAFFIC_FILE):
        prev = json.load(open(TRAFFIC_FILE)).get("kernels", {})
    prev.update(out["kernels"])
    # records taken on sources that have changed since describe kernels that no longer exist
    out["kernels"] = {k: r for k, r in prev.items()
                      if r.get("source_hash") == kernel_source_hash(k.split("@")[0])}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(w, threads, gpu_o, gpu_f):
    import oracle
    inp = synth.oracle_inputs(w)
    pairs = [(n, h) for n in range(w.N) for h in range(w.H)]
    t0 = time.perf_counter()
    ro, rf = oracle.kda_forward(**inp, pairs=pairs, threads=threads)
    dt = time.perf_counter() - t0
    par_o = synth.parity(gpu_o, ro)
    par_f = synth.parity(gpu_f, rf)
    return dt, par_o, par_f, rf


def cpu_one_thread(w, chains):
    """The oracle on one thread over the first ``chains`` (sequence, head) chains: seconds."""
    import oracle
    inp = synth.oracle_inputs(w)
    pairs = [(n, h) for n in range(w.N) for h in range(w.H)][:chains]
    t0 = time.perf_counter()
    oracle.kda_forward(**inp, pairs=pairs, threads=1)
    return time.perf_counter() - t0, pairs


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(args, dev):
    """A plain device copy of known size: the reference for the HBM byte counters."""
    import torch

    if not args.copy_calibration:
        return
    nbytes = args.copy_calibration << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 x {nbytes} bytes read + written")


def bench_decode(args, dev):
    """Decode step: N sequences, one token each, state updated in place every step."""
    import torch
    import chunked_gated_delta_kda_amd as kda

    N, H = args.decode, args.heads
    bf16 = args.state_dtype == "bf16"
    log(f"[bench] decode: {N} sequences x {H} heads, {args.state_dtype} state")
    w = synth.make_workload([1] * N, H, 1000 + N, with_initial_state=True)
    w.initial_state *= np.float32(3.0)     # a state of the size a long prefill leaves (RMS ~0.06)
    if bf16:   # the drawn state rounded to bf16; the oracle starts from the same values
        bits = synth.bf16_bits(w.initial_state)
        w.initial_state = synth.bf16_to_f32(bits)
        s0 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    d = synth.to_device(w, dev)
    if not bf16:
        s0 = d["initial_state"]
    q, k, v, g, beta = d["q"], d["k"], d["v"], d["g"], d["beta"]
    # parity of one step from the drawn state (written to a separate buffer)
    o1, s1 = kda.decode(q, k, v, g, beta, w.scale, s0, state_out=torch.empty_like(s0))
    torch.cuda.synchronize()
    o1, s1 = o1.cpu().numpy(), s1.float().cpu().numpy()
    state = s0.clone()
    out = torch.empty((N, H, 128), dtype=torch.float32, device=dev)

    def step():
        kda.decode(q, k, v, g, beta, w.scale, state, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    with no_gc():
        t0 = time.perf_counter()
        for a, b in evs:
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    copy_calibration(args, dev)
    alg_bytes = N * H * (2 * STATE_BYTES // (2 if bf16 else 1) + 1796)
    achieved = alg_bytes / (launch_ms / 1e3) / 1e9
    res = {"metric": DECODE_METRIC, "value": round(N / (ms_per_step / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": f"synthetic (seeded; bf16 q/k/v, fp32 g/beta, {args.state_dtype} state)",
           "config": {"workload": f"decode step, {N} sequences x {H} heads, {args.state_dtype} state", "num_seqs": N,
                      "num_heads": H, "dk": 128, "dv": 128, "state_dtype": args.state_dtype},
           "roofline": {"bound": "hbm", "kernel": "recurrent", "achieved": round(achieved, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("recurrent", f"decode{N}x{H}" + ("bf16" if bf16 else "")),
                        "alg_bytes_per_launch": alg_bytes, "launches_per_step": 1,
                        "avg_launch_ms": round(launch_ms, 5)},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle
        inp = synth.oracle_inputs(w)
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            cores = os.cpu_count() or 1
        threads = args.cpu_threads or min(16, cores)
        t0 = time.perf_counter()
        ro, rf = oracle.kda_forward(**inp, threads=threads)
        dt = time.perf_counter() - t0
        po = synth.parity(o1, ro)
        pf = synth.parity_bf16(s1, rf) if bf16 else synth.parity(s1, rf)
        res["cpu_baseline"] = {"value": round(N / dt, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"one decode step of the whole batch ({N * H} (sequence, head) "
                                         f"states), fp64, {dt:.3f} s wall"}
        fkeys = ("rel_l2", "max_abs_rms") + (("max_err_over_bf16_bound",) if bf16 else ())
        res["parity"] = {"o": {k: po[k] for k in ("rel_l2", "max_abs_rms")},
                         "final_state": {k: pf[k] for k in fkeys},
                         "pass": synth.passes(po) and (synth.passes_bf16(pf) if bf16 else synth.passes(pf))}
    print(json.dumps(res), flush=True)


BWD_METRIC = "KDA backward (all gradients) tokens/s, 1 MI355X (dk=dv=128)"
# Algorithmic bytes of the backward per token-head: q, k, v bf16 (3 x 256) + g, d_out fp32
# (2 x 512) + beta (4) read; dq, dk, dv, dg fp32 (4 x 512) + dbeta (4) written. Plus 64 KiB
# per (sequence, head) for the initial state, the final-state gradient and d_initial_state.
BWD_BYTES_PER_TOKEN_HEAD = 3 * 256 + 2 * 512 + 4 + 4 * 512 + 4
# Algorithmic fp32 operations of the backward per token-head, per element of the 128 x 128
# state (terms per row or column alone are negligible): the forward step it differentiates
# (decay 1 multiply, u = S1^T k 1 FMA, S = S1 + k d^T 1 FMA: 5 flops) and the reverse step
# (dS += scale q do^T, dq's S1 do, dd = dS^T k, dk's dS d and S1 du, dS1 = dS + k du^T,
# dg's row sum of S1 * dS1: 7 FMAs; dS_prev = e * dS1: 1 multiply: 15 flops).
BWD_FLOP_PER_TOKEN_HEAD = 20 * 128 * 128
# fp32 vector peak of MI355X (256 CUs at 2.4 GHz, 256 flops per CU per clock with packed FMA);
# without packed fp32 instructions (not used here) a kernel's ceiling is half of it
FP32_VECTOR_PEAK_TFLOPS = 157.3


def bench_backward(args, dev, cfg=None, cpu=True):
    """Backward step: kda_bwd over the whole --config (or cfg) workload per step; returns the
    result dict."""
    import torch
    import chunked_gated_delta_kda_amd as kda

    cfg = args.config if cfg is None else cfg
    log(f"[bench] backward, config {cfg}: {synth.CONFIGS[cfg]['name']}")
    w = synth.config_workload(cfg)
    d = synth.to_device(w, dev)
    rng = np.random.Generator(np.random.PCG64(5000 + cfg))
    do_h = rng.standard_normal((w.T, w.H, 128)).astype(np.float32)
    dsf_h = rng.standard_normal((w.N, w.H, 128, 128)).astype(np.float32) * np.float32(0.1)
    do, dsf = torch.from_numpy(do_h).to(dev), torch.from_numpy(dsf_h).to(dev)
    ws = torch.empty(kda.native.load_library().kda_bwd_workspace_bytes(w.N, w.T, w.H), dtype=torch.uint8,
                     device=dev)

    def step():
        return kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["scale"], d["cu_seqlens"],
                       d["initial_state"], dsf, workspace=ws)

    for _ in range(args.warmup):
        gr = step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    with no_gc():
        t0 = time.perf_counter()
        for a, b in evs:
            a.record()
            gr = step()
            b.record()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    alg = w.T * w.H * BWD_BYTES_PER_TOKEN_HEAD + w.N * w.H * STATE_BYTES * (3 if w.initial_state is not None else 2)
    achieved = alg / (call_ms / 1e3) / 1e9
    alg_flops = w.T * w.H * BWD_FLOP_PER_TOKEN_HEAD
    tflops = alg_flops / (call_ms / 1e3) / 1e12
    res = {"metric": BWD_METRIC, "value": round(w.T / (ms_per_step / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded; bf16 q/k/v, fp32 g/beta/d_out/final-state gradient)",
           "config": {"workload": synth.CONFIGS[cfg]["name"] + ", backward", "num_seqs": w.N,
                      "total_tokens": w.T, "num_heads": w.H, "dk": 128, "dv": 128},
           # the backward is bound by vector arithmetic (a token loop in fp32 registers), not
           # by HBM: its roofline is the fp32 vector peak; the HBM figure is kept beside it
           "roofline": {"bound": "alu", "kernel": "bwd", "achieved": round(tflops, 2),
                        "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                        "alg_flops_per_launch": alg_flops, "avg_call_ms": round(call_ms, 4),
                        "hbm": {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(achieved / HBM_PEAK_GBS, 5), "alg_bytes_per_launch": alg}},
           "cpu_baseline": None}
    if cpu and not args.no_cpu_baseline:
        import oracle
        # the first two chains of the first sequence, on the oracle (one thread each)
        n_tok = int(w.cu_seqlens[1])
        heads = [0, 1] if w.H > 1 else [0]
        sub = dict(q=w.q_f32()[:n_tok, heads].astype(np.float64), k=w.k_f32()[:n_tok, heads].astype(np.float64),
                   v=w.v_f32()[:n_tok, heads].astype(np.float64), g=w.g[:n_tok, heads].astype(np.float64),
                   beta=w.beta[:n_tok, heads].astype(np.float64), scale=float(w.scale),
                   cu_seqlens=np.array([0, n_tok], dtype=np.int64),
                   initial_state=None if w.initial_state is None else w.initial_state[:1, heads].astype(np.float64))
        t0 = time.perf_counter()
        ref = oracle.kda_backward(**sub, d_out=do_h[:n_tok, heads], d_final_state=dsf_h[:1, heads],
                                  threads=len(heads))
        dt = time.perf_counter() - t0
        got = {n: gr[n].cpu().numpy() for n in ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")}
        par = {}
        ok = True
        for n, v in got.items():
            v = v[:1, heads] if n == "d_initial_state" else v[:n_tok, heads]
            m = synth.parity(v, ref[n])
            par[n] = {k: m[k] for k in ("rel_l2", "max_abs_rms")}
            ok &= synth.passes(m)
        par["pass"] = ok
        res["parity"] = par
        th = n_tok * len(heads)
        res["cpu_baseline"] = {"value": round(th / dt / w.H, 1), "unit": "tokens/s", "cores": len(heads),
                               "kind": "oracle",
                               "sample": f"{len(heads)} of {w.N * w.H} chains ({th} token-heads), fp64, "
                                         f"{dt:.2f} s wall, scaled to tokens of {w.H} heads"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=sorted(synth.CONFIGS),
                    help="workload (default 2: fixed-length prefill T=8192, H=32)")
    ap.add_argument("--variant", default="auto", choices=["auto", "split", "fused", "recurrent"])
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="benchmark the decode step over N sequences instead of a prefill config")
    ap.add_argument("--heads", type=int, default=32, help="heads of the --decode workload")
    ap.add_argument("--backward", action="store_true",
                    help="benchmark the backward (kda_bwd) over the --config workload instead")
    ap.add_argument("--state-dtype", default="f32", choices=["f32", "bf16"],
                    help="state element type in HBM (bf16: the BF16-state form; prefill initial/final "
                         "state or the --decode state)")
    ap.add_argument("--g-dtype", default="f32", choices=["f32", "bf16"],
                    help="element type of g for the prefill (bf16: the input-byte diet form)")
    ap.add_argument("--no-gated", action="store_true",
                    help="do not also time the T=8192 varlen workload (config 3) after the headline one")
    ap.add_argument("--no-others", action="store_true",
                    help="do not also time the other prefill workloads (configs 1, 4, 5) and the backward "
                         "on config 3 after the headline one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: host cores, max 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (3 times) after the timed steps, "
                         "as the reference kernel for HBM byte counters")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 counter runs and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --ingest-pmc")
    args = ap.parse_args()

    if args.ingest_pmc:
        workload = (f"decode{args.decode}x{args.heads}" + ("bf16" if args.state_dtype == "bf16" else "")
                    if args.decode else f"config{args.config}" + ("_bf16g" if args.g_dtype == "bf16" else "")
                    + ("_bf16state" if args.state_dtype == "bf16" else ""))
        ingest_pmc(*args.ingest_pmc, workload, args.pmc_command)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.decode:
        bench_decode(args, dev)
        return
    if args.backward:
        print(json.dumps(bench_backward(args, dev)), flush=True)
        return
    res = run_prefill(args.config, args, dev, cpu=not args.no_cpu_baseline)
    if args.config != GATED_CONFIG and not args.no_gated:
        g = run_prefill(GATED_CONFIG, args, dev, cpu=False)
        res["gated_config"] = {k: g[k] for k in ("config", "value", "unit", "ms_per_step", "cold", "kernel_ms",
                                                 "roofline", "path_hbm_frac")}
        res["gated_config"]["bar_ms"] = GATED_BAR_US / 1e3
    if not args.no_others:
        # the other prefill workloads and the backward, each timed as above (no CPU leg)
        others = {}
        for cfg in OTHER_CONFIGS:
            if cfg in (args.config, GATED_CONFIG):
                continue
            o = run_prefill(cfg, args, dev, cpu=False)
            others[f"config{cfg}"] = {k: o[k] for k in ("config", "value", "unit", "ms_per_step", "cold")}
        res["other_configs"] = others
        b = bench_backward(args, dev, cfg=GATED_CONFIG, cpu=False)
        res["backward"] = {k: b[k] for k in ("metric", "value", "unit", "ms_per_step", "config", "roofline")}
        res["backward"]["avg_call_ms"] = b["roofline"]["avg_call_ms"]
    print(json.dumps(res), flush=True)


def run_prefill(cfg, args, dev, cpu):
    """Time one prefill workload (kda_fwd over the whole batch per step); returns the result dict."""
    import torch
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import native

    log(f"[bench] generating config {cfg}: {synth.CONFIGS[cfg]['name']}")
    w = synth.config_workload(cfg)
    g_bf16, s_bf16 = args.g_dtype == "bf16", args.state_dtype == "bf16"
    if g_bf16:       # the input-byte diet forms run on the bf16-rounded values
        w.g = synth.bf16_to_f32(synth.bf16_bits(w.g))
    if s_bf16 and w.initial_state is not None:
        w.initial_state = synth.bf16_to_f32(synth.bf16_bits(w.initial_state))
    d = synth.to_device(w, dev)
    sdt = torch.bfloat16 if s_bf16 else torch.float32
    if g_bf16:
        d["g"] = d["g"].to(torch.bfloat16)
    if s_bf16 and d["initial_state"] is not None:
        d["initial_state"] = d["initial_state"].to(torch.bfloat16)
    N, T, H = w.N, w.T, w.H
    variant = args.variant if args.variant != "auto" else kda.select_variant(N, T, H)
    out = torch.empty((T, H, 128), dtype=torch.float32, device=dev)
    fin = torch.empty((N, H, 128, 128), dtype=sdt, device=dev)
    nws = kda.workspace_bytes(N, T, H, variant)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    launch_info = native.launch_plan(N, T, H, variant)
    plan = [p[0] for p in launch_info]
    chunk_len = launch_info[0][3]
    if (g_bf16 or s_bf16) and variant == "split" and chunk_len != 32:
        log("[bench] note: bf16 inputs run the 32-token forms; the launch plan shown is the fp32 one")
    names = list(dict.fromkeys(plan))            # kinds, first-launch order
    ev = HipEvents()
    n_ev = len(plan) + 1
    step_events = [ev.array(n_ev) if i % EVENT_EVERY == 0 else None for i in range(args.steps)]

    def step(events=None):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["cu_seqlens"],
                d["initial_state"], variant=variant, out=out, final_state=fin, workspace=ws,
                stage_events=events, state_dtype=sdt)

    log(f"[bench] variant={variant} warmup={args.warmup} steps={args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    with no_gc():
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(step_events[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = {nm: 0.0 for nm in names}
    sampled = [e for e in step_events if e is not None]
    for j, nm in enumerate(plan):
        kern_ms[nm] += float(np.mean([ev.ms(e[j], e[j + 1]) for e in sampled]))
    launches = {nm: plan.count(nm) for nm in names}
    ev.close()
    # cold caches: each step after a 512 MiB write that evicts L2 and MALL (HIP events around
    # the call only, on the stream the library uses)
    flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(COLD_STEPS):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    copy_calibration(args, dev)
    log(f"[bench] {ms_per_step:.4f} ms/step; kernels (ms summed over launches): {kern_ms}; "
        f"launches {launches}")

    TH = T * H
    unit = BYTES_PER_TOKEN_HEAD - (256 if g_bf16 else 0)
    state_b = STATE_BYTES // (2 if s_bf16 else 1)
    states = N * H * state_b * ((1 if w.initial_state is not None else 0) + 1)
    alg_bytes_total = TH * unit + states
    alg_flops = TH * FLOP_PER_TOKEN_HEAD
    step_s = ms_per_step / 1e3
    tokens_per_s = T / step_s

    # token counts per segment (a fraction of every sequence's chunks), from the lengths
    cl = chunk_len
    seg_one = native.SEGMENT_ONE
    seq_csum = [np.concatenate([[0], np.cumsum(np.minimum(cl, L - cl * np.arange((L + cl - 1) // cl)))])
                for L in w.lengths]

    def tokens_in(r):
        t = 0
        for cs in seq_csum:
            c = len(cs) - 1
            a, b = c * r[0] // seg_one, c * r[1] // seg_one
            t += int(cs[b] - cs[a]) if b > a else 0
        return t

    def launch_bytes(kind, prep_r, recur_r):
        """(algorithmic bytes credited to one launch, bytes of its own inputs and outputs):
        the unit's bytes for every token-head the launch processes; the batch's states
        with the last recurrence launch (or the one-launch kinds)."""
        if kind == "chunk_map":
            b = 4 * (N + 1) + 8 * N
            return b, b
        if kind in ("fused", "recurrent", "parts"):
            own = TH * (KERNEL_OWN_BYTES_PER_TOKEN_HEAD["recur"] if kind == "parts" else unit) + states
            return TH * unit + states, own
        tp, tr = tokens_in(prep_r) * H, tokens_in(recur_r) * H
        own = (tp * (KERNEL_OWN_BYTES_PER_TOKEN_HEAD["prep"] - (256 if g_bf16 else 0))
               + tr * KERNEL_OWN_BYTES_PER_TOKEN_HEAD["recur"])
        alg = max(tp, tr) * unit
        if recur_r[1] == seg_one and recur_r[1] > recur_r[0]:
            alg += states
            own += states
        return alg, own

    kind_bytes = {nm: 0 for nm in names}
    own_bytes = {nm: 0 for nm in names}
    for kind, pr, rr, _ in launch_info:
        a_b, o_b = launch_bytes(kind, pr, rr)
        kind_bytes[kind] += a_b
        own_bytes[kind] += o_b

    dom = max((nm for nm in names if nm != "chunk_map"), key=lambda nm: kern_ms[nm])
    dom_s = kern_ms[dom] / 1e3
    achieved = kind_bytes[dom] / dom_s / 1e9
    workload = f"config{cfg}" + ("_bf16g" if g_bf16 else "") + ("_bf16state" if s_bf16 else "")
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, workload),
                "alg_bytes_per_launch": int(kind_bytes[dom] / launches[dom]),
                "own_bytes_per_launch": int(own_bytes[dom] / launches[dom]),
                "launches_per_step": launches[dom],
                "avg_launch_ms": round(kern_ms[dom] / launches[dom], 5)}

    res = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; bf16 q/k/v, " + ("bf16" if g_bf16 else "fp32") + " g, fp32 beta)",
           "config": {"workload": f"{synth.CONFIGS[cfg]['name']} (config {cfg})",
                      "num_seqs": N, "total_tokens": T, "num_heads": H, "dk": 128, "dv": 128,
                      "chunk": chunk_len, "variant": variant, "initial_state": w.initial_state is not None,
                      "g_dtype": args.g_dtype, "state_dtype": args.state_dtype},
           "tflops": round(alg_flops / step_s / 1e12, 2),
           "mfma_bf16_peak_frac": round(alg_flops / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "path_hbm_frac": round(alg_bytes_total / step_s / 1e9 / HBM_PEAK_GBS, 4),
           "kernel_ms": {k: round(v, 5) for k, v in kern_ms.items()},
           "cold": {"ms_per_step_median": round(float(np.median(cold)), 5),
                    "tokens_per_s": round(T / (float(np.median(cold)) / 1e3), 1), "steps": COLD_STEPS,
                    "flush_bytes_before_each": COLD_FLUSH_BYTES},
           "kernel_launches": launches,
           "roofline": roofline, "cpu_baseline": None}

    if cpu:
        try:
            host = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            host = os.cpu_count() or 1
        # the machine's CPU share for one GPU is 16 threads, whatever the host shows
        threads = args.cpu_threads or min(16, host)
        log(f"[bench] oracle on the host: {N * H} chains, {threads} threads")
        o_np = out.cpu().numpy()
        f_np = fin.float().cpu().numpy()
        dt, po, pf, rf = cpu_baseline(w, threads, o_np, f_np)
        one = min(4, N * H)
        dt1, pairs1 = cpu_one_thread(w, one)
        th1 = int(sum(w.lengths[n] for n, _ in pairs1))
        res["cpu_baseline"] = {"value": round(T / dt, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole workload ({N * H} (sequence, head) chains, "
                                         f"{TH} token-heads), fp64 token loop, {dt:.2f} s wall",
                               "cpu_model": cpu_model(), "host_cpus": host,
                               "one_thread": {"token_heads_per_s": round(th1 / dt1, 1),
                                              "sample": f"{one} chains ({th1} token-heads), {dt1:.2f} s"}}
        if s_bf16:   # a bf16 final state: the bf16-result gate
            pf = synth.parity_bf16(f_np, rf, synth.GATE_MAX_ABS_RMS)
        ok_f = synth.passes_bf16(pf) if s_bf16 else synth.passes(pf)
        res["parity"] = {"o": {k: po[k] for k in ("rel_l2", "max_abs_rms")},
                         "final_state": {k: pf[k] for k in ("rel_l2", "max_abs_rms")},
                         "pass": synth.passes(po) and ok_f}
    return res


if __name__ == "__main__":
    main()

"""Seeded synthetic KDA workloads and the parity gate.

This module holds no KDA arithmetic: it draws inputs (the distributions are
the ones the workload descriptions fix) and measures the distance between two
outputs. Tests, the benchmark and the smoke check draw their inputs here, and
the same host arrays feed both the GPU path and the fp64 oracle.

Recipe (every workload): q, k ~ N(0,1) fp32, L2-normalised over the 128
channels of each (token, head), then rounded to bf16 (round-to-nearest-even);
v ~ N(0,1) rounded to bf16; g = max(-softplus(z), -5) fp32 with z ~ N(0,1);
beta = sigmoid(z') fp32; scale = fp32(1/sqrt(128)). Draw order: lengths,
q, k, v, g normals, clamp mask, beta normals, initial state.
"""
from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 128
LOWER_BOUND = -5.0

#: Parity gate on o and on final_state (each against the fp64 oracle):
#: relative L2 error and max-abs error measured in units of the oracle's RMS.
GATE_REL_L2 = 1e-2
GATE_MAX_ABS_RMS = 2e-2


# ----------------------------------------------------------------------------- bf16 helpers
def bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    q: np.ndarray          # uint16 bf16 bits [T, H, D]
    k: np.ndarray          # uint16 bf16 bits [T, H, D]
    v: np.ndarray          # uint16 bf16 bits [T, H, D]
    g: np.ndarray          # float32 [T, H, D]
    beta: np.ndarray       # float32 [T, H]
    cu_seqlens: np.ndarray  # int32 [N+1]
    initial_state: np.ndarray = None  # float32 [N, H, D, D] or None
    scale: float = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def N(self):
        return self.cu_seqlens.shape[0] - 1

    @property
    def lengths(self):
        return np.diff(self.cu_seqlens.astype(np.int64))

    def q_f32(self):
        return bf16_to_f32(self.q)

    def k_f32(self):
        return bf16_to_f32(self.k)

    def v_f32(self):
        return bf16_to_f32(self.v)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _unit_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _softplus(z):
    return np.logaddexp(np.float32(0.0), z).astype(np.float32)


def make_workload(lengths, H, seed, *, with_initial_state=False, clamp_frac=0.0, D=HEAD_DIM,
                  name="custom", rng=None):
    """Draw one workload with the given sequence lengths (lengths already drawn)."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.ndim == 1 and lengths.size >= 1 and (lengths >= 0).all()
    T = int(lengths.sum())
    cu = np.zeros(lengths.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q = bf16_bits(_unit_rows(_normal(rng, (T, H, D))))
    k = bf16_bits(_unit_rows(_normal(rng, (T, H, D))))
    v = bf16_bits(_normal(rng, (T, H, D)))
    g = np.maximum(-_softplus(_normal(rng, (T, H, D))), np.float32(LOWER_BOUND)).astype(np.float32)
    if clamp_frac > 0.0:
        mask = rng.random((H, D)) < clamp_frac          # fixed over time, per (head, channel)
        g[:, mask] = np.float32(LOWER_BOUND)
    beta = (1.0 / (1.0 + np.exp(-_normal(rng, (T, H)).astype(np.float64)))).astype(np.float32)
    s0 = None
    if with_initial_state:
        s0 = (_normal(rng, (lengths.size, H, D, D)) * np.float32(0.02)).astype(np.float32)
    return Workload(name=name, q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, initial_state=s0,
                    meta={"seed": seed, "clamp_frac": clamp_frac})


def skewed_lengths(rng, n=12, total=32768, lo=37, hi=16384):
    """Log-uniform lengths in [lo, hi] rescaled to ``total`` tokens (floor, min 1,
    deficit to the longest); if every length is a multiple of 16, move one token."""
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    e = np.exp(u)
    L = np.maximum(np.floor(e * total / e.sum()).astype(np.int64), 1)
    L[np.argmax(L)] += total - L.sum()
    if np.all(L % 16 == 0):
        L[0] -= 1
        L[1] += 1
    return L


CONFIGS = {
    1: dict(name="tiny T=256 H=2", lengths=[256], H=2, init=False, clamp=0.0),
    2: dict(name="fixed-length prefill T=8192 H=32", lengths=[8192], H=32, init=False, clamp=0.0),
    3: dict(name="uniform varlen 8x1024 H=16", lengths=[1024] * 8, H=16, init=True, clamp=0.0),
    4: dict(name="long context T=65536 H=8", lengths=[65536], H=8, init=False, clamp=0.1),
    5: dict(name="skewed varlen 12 seqs T=32768 H=32", lengths=None, H=32, init=True, clamp=0.0),
}


def config_workload(idx):
    """The five benchmark workloads; seed = config index."""
    c = CONFIGS[idx]
    rng = np.random.Generator(np.random.PCG64(idx))
    lengths = c["lengths"] if c["lengths"] is not None else skewed_lengths(rng)
    return make_workload(lengths, c["H"], idx, with_initial_state=c["init"], clamp_frac=c["clamp"],
                         name=c["name"], rng=rng)


def config_token_heads(idx):
    c = CONFIGS[idx]
    T = 32768 if c["lengths"] is None else int(sum(c["lengths"]))
    return T * c["H"]


# ----------------------------------------------------------------------------- parity gate
def parity(got, ref):
    """Distance of ``got`` from the fp64 reference ``ref``.

    rel_l2 = ||got - ref||_2 / ||ref||_2 ; max_abs_rms = max|got - ref| / RMS(ref).
    When ref is identically zero, both are reported as max|got| (so only an exact
    zero passes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return {"rel_l2": 0.0, "max_abs_rms": 0.0, "rms": 0.0, "finite": True}
    finite = bool(np.isfinite(got).all())
    err = got - ref
    nref = float(np.sqrt(np.sum(ref * ref)))
    rms = nref / math.sqrt(ref.size)
    if nref == 0.0:
        m = float(np.max(np.abs(got))) if finite else float("inf")
        return {"rel_l2": m, "max_abs_rms": m, "rms": 0.0, "finite": finite}
    return {"rel_l2": float(np.sqrt(np.sum(err * err))) / nref if finite else float("inf"),
            "max_abs_rms": float(np.max(np.abs(err))) / rms if finite else float("inf"),
            "rms": rms, "finite": finite}


def passes(m, rel=GATE_REL_L2, mx=GATE_MAX_ABS_RMS):
    return m["finite"] and m["rel_l2"] <= rel and m["max_abs_rms"] <= mx


#: A result stored in bf16 is at best the rounding of the exact value (error up to half a
#: bf16 ulp, 2^-9 |x|): on top of the relative-L2 gate, every element must lie within one
#: bf16 ulp (bounded by 2^-7 |ref|) of the fp64 reference, plus an absolute allowance for
#: the fp32 arithmetic before the rounding: 1e-4 RMS for the decode step's fp32 update
#: (GATE_BF16_ABS_RMS); for the prefill's final state, whose fp32 value carries the split
#: products of the chunked form, the fp32 result's own max-abs gate (GATE_MAX_ABS_RMS).
GATE_BF16_ULP = 2.0 ** -7
GATE_BF16_ABS_RMS = 1e-4


def parity_bf16(got, ref, abs_rms=GATE_BF16_ABS_RMS):
    """``parity`` plus the largest elementwise error in units of the bf16 bound."""
    m = parity(got, ref)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = GATE_BF16_ULP * np.abs(ref) + abs_rms * m["rms"]
    m["max_err_over_bf16_bound"] = float(np.max(np.abs(got - ref) / bound)) if ref.size and m["finite"] else 0.0
    return m


def passes_bf16(m, rel=GATE_REL_L2):
    return m["finite"] and m["rel_l2"] <= rel and m["max_err_over_bf16_bound"] <= 1.0


# ----------------------------------------------------------------------------- device upload
def to_device(w, device="cuda"):
    """Copy a workload's host arrays to device tensors (bf16 bits are reinterpreted, not converted)."""
    import torch

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)

    d = {"q": bf16(w.q), "k": bf16(w.k), "v": bf16(w.v),
         "g": torch.from_numpy(w.g).to(device), "beta": torch.from_numpy(w.beta).to(device),
         "cu_seqlens": torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(device),
         "initial_state": None if w.initial_state is None else torch.from_numpy(w.initial_state).to(device),
         "scale": w.scale}
    return d


def oracle_inputs(w):
    """The same inputs as float64 host arrays (exact upcast), for the oracle."""
    return dict(q=w.q_f32().astype(np.float64), k=w.k_f32().astype(np.float64),
                v=w.v_f32().astype(np.float64), g=w.g.astype(np.float64),
                beta=w.beta.astype(np.float64), scale=float(w.scale),
                cu_seqlens=w.cu_seqlens.astype(np.int64),
                initial_state=None if w.initial_state is None else w.initial_state.astype(np.float64))

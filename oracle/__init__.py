"""KDA forward oracle -- TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU token-by-token evaluation of the Kimi Delta Attention
recurrence (see kda_oracle.c for the formula and the readings it takes).
Only tests/, the package smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP path.

``kda_forward`` takes numpy arrays of any real dtype; they are upcast to
float64 exactly (bf16/fp32 values are exactly representable in fp64).
"""
import ctypes
import os

import numpy as np

from .build import LIB, build as _build

__all__ = ["kda_forward", "kda_backward", "LOWER_BOUND", "load_library"]

#: log-decay clamp the FlashKDA articles state (smzdm "KDA 内核到底难在哪").
LOWER_BOUND = -5.0

_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            _build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double, ip,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   dp, ctypes.c_double, dp, dp, ip, ctypes.c_int64, ctypes.c_int]
    if hasattr(lib, "kda_oracle_bwd"):
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double, ip,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       dp, ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(typ))


def default_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def kda_forward(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None,
                lower_bound=LOWER_BOUND, pairs=None, threads=None, lib=None):
    """Run the fp64 token-loop oracle.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H, dk]; beta: [T, H];
    cu_seqlens: [N+1] (None = one sequence of length T);
    initial_state: [N, H, dk, dv] or None (zeros);
    pairs: optional iterable of (n, h) chains to evaluate (others left 0).
    Returns (o [T, H, dv], final_state [N, H, dk, dv]) as float64.
    """
    lib = lib or load_library()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert cu[-1] == T
    s0 = None
    if initial_state is not None:
        s0 = _f64(initial_state)
        assert s0.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    pr = None
    n_pairs = 0
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(list(pairs), dtype=np.int64).reshape(-1, 2))
        n_pairs = pr.shape[0]
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                            _ptr(cu, ctypes.c_int64), N, H, dk, dv, _ptr(s0), float(lower_bound),
                            _ptr(out), _ptr(fin), _ptr(pr, ctypes.c_int64), n_pairs,
                            int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"kda_oracle_fwd failed with code {rc}")
    return out, fin


def kda_backward(q, k, v, g, beta, scale, d_out, cu_seqlens=None, initial_state=None, d_final_state=None,
                 lower_bound=LOWER_BOUND, threads=None, lib=None):
    """Gradients of the forward oracle's outputs (fp64 reverse-mode token loop).

    d_out: [T, H, dv] gradient of o; d_final_state: [N, H, dk, dv] or None (zero).
    Returns dict(dq [T,H,dk], dk [T,H,dk], dv [T,H,dv], dg [T,H,dk], dbeta [T,H],
    d_initial_state [N,H,dk,dv]) as float64 (d_initial_state is the gradient with respect
    to the initial state, zeros standing in when none was given).
    """
    lib = lib or load_library()
    q, k, v, g, beta, d_out = map(_f64, (q, k, v, g, beta, d_out))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert d_out.shape == (T, H, dv)
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    s0 = None if initial_state is None else _f64(initial_state)
    dfin = None if d_final_state is None else _f64(d_final_state)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dg=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)), d_initial_state=np.zeros((N, H, dk, dv)))
    rc = lib.kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                            _ptr(cu, ctypes.c_int64), N, H, dk, dv, _ptr(s0), float(lower_bound),
                            _ptr(d_out), _ptr(dfin), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["d_initial_state"]),
                            int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"kda_oracle_bwd failed with code {rc}")
    return out

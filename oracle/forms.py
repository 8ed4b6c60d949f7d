"""Independent fp64 forms of the KDA forward, used only to pin the oracle.

TEST INFRASTRUCTURE ONLY. None of this is called by the GPU path.

* ``matrix_form``: the recurrence written with explicit dk x dk matrices,
  S_t = (I - b k k^T) Diag(e^g) S_{t-1} + b k v^T, o_t = scale S_t^T q_t
  (O(dk^2 dv) per token; for tiny sizes). The delta-rule-with-gate form the
  FlashKDA articles describe (smzdm "KDA 内核到底难在哪").
* ``chunked_form``: the chunk-parallel rewrite the articles credit for making
  the recurrence tensor-core friendly (16-token chunks, one state chain across
  chunks; smzdm "KDA 内核到底难在哪"). Inside a chunk the per-token corrections
  solve a unit lower-triangular system (I + A) X = Diag(b)(V - K^+ S_0), here
  solved by forward substitution or by the Neumann product
  (I - A)(I + A^2)(I + A^4)(I + A^8), which is exact because A^16 = 0.
  Optionally the decay factors are anchored at the chunk midpoint (the
  exponent-centring scalar the B200 section describes, smzdm "反转二"): the
  anchor cancels in every product, so results agree to rounding.
"""
import numpy as np


def _clamped(g, lower_bound):
    return np.maximum(g, lower_bound) if lower_bound is not None else g


def _seqs(T, cu_seqlens):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    return np.asarray(cu_seqlens, dtype=np.int64)


def matrix_form(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, lower_bound=-5.0):
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _seqs(T, cu_seqlens)
    N = len(cu) - 1
    g = _clamped(g, lower_bound)
    o = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    eye = np.eye(dk)
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            for t in range(cu[n], cu[n + 1]):
                kt = k[t, h][:, None]
                M = (eye - beta[t, h] * (kt @ kt.T)) @ np.diag(np.exp(g[t, h]))
                S = M @ S + beta[t, h] * (kt @ v[t, h][None, :])
                o[t, h] = scale * (S.T @ q[t, h])
            fin[n, h] = S
    return o, fin


def _unit_lower_inverse_subst(A):
    """(I + A)^{-1} for strictly lower-triangular A, by forward substitution."""
    n = A.shape[0]
    X = np.zeros((n, n))
    for r in range(n):
        row = np.zeros(n)
        row[r] = 1.0
        for s in range(r):
            row -= A[r, s] * X[s]
        X[r] = row
    return X


def _unit_lower_inverse_neumann(A):
    """(I + A)^{-1} = sum_j (-A)^j, grouped by repeated squaring (A nilpotent)."""
    n = A.shape[0]
    eye = np.eye(n)
    X = eye - A
    P = A @ A
    m = 2
    while m < n:
        X = X @ (eye + P)
        P = P @ P
        m *= 2
    return X


def chunked_form(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, lower_bound=-5.0,
                 chunk=16, inverse="subst", anchor=False):
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _seqs(T, cu_seqlens)
    N = len(cu) - 1
    g = _clamped(g, lower_bound)
    inv = {"subst": _unit_lower_inverse_subst, "neumann": _unit_lower_inverse_neumann}[inverse]
    o = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                Q, K, V, b = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h], axis=0)          # in-chunk cumulative log decay
                a = G[(c1 - c0) // 2] if anchor else np.zeros(dk)
                Kp, Km, Qp = K * np.exp(G - a), K * np.exp(a - G), Q * np.exp(G - a)
                Qs = Q * np.exp(G)                           # for the read of S_0
                Kw = K * np.exp(G)                           # for the correction against S_0
                A = b[:, None] * np.tril(Kp @ Km.T, -1)
                Tm = inv(A)
                W = Tm @ (b[:, None] * Kw)
                U = Tm @ (b[:, None] * V)
                Vn = U - W @ S                               # true per-token writes u_t
                P = np.tril(Qp @ Km.T)                       # causal, diagonal included
                o[c0:c1, h] = scale * (Qs @ S + P @ Vn)
                GC = G[-1]
                S = np.exp(GC)[:, None] * S + (K * np.exp(GC - G)).T @ Vn
            fin[n, h] = S
    return o, fin

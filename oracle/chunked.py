"""Chunk-parallel (WY) form of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

An independent derivation of the same result as :func:`oracle.gdn_serial`,
used to cross-check it (the chunked and token-serial forms must agree to
rounding). It follows the chunk-parallel form that the "GDN CTE Kernel API
Reference" page describes in its introduction (work inside a chunk is done in
parallel through a triangular inverse, a recurrence runs across chunks); the
page gives no formulas, the ones below are derived from the recurrence.

For one head and one chunk of C tokens with start state S0 and
gamma_r = sum_{i<=r} g_i (within-chunk inclusive cumulative log decay):

    A[r,s] = beta_r (k_r . k_s) e^{gamma_r - gamma_s}   for s < r, else 0
    T      = (I + A)^{-1}                 (unit lower-triangular inverse)
    W      = T diag(beta e^gamma) K       [C, Dk]
    U~     = T diag(beta) V               [C, Dv]
    U      = U~ - W S0                    [C, Dv]  (the per-token updates u_t)
    O      = scale (diag(e^gamma) Q S0 + (Q K^T (.) M) U),
             M[r,s] = e^{gamma_r - gamma_s} for s <= r, else 0
    S_C    = e^{gamma_C} S0 + (diag(e^{gamma_C - gamma}) K)^T U

Derivation: with u_t = beta_t (v_t - e^{g_t} S_{t-1}^T k_t) the recurrence is
S_t = e^{g_t} S_{t-1} + k_t u_t^T, so S_r = e^{gamma_r} S0 + sum_{s<=r}
e^{gamma_r - gamma_s} k_s u_s^T; substituting S_{r-1} into u_r gives
(I + A) U = diag(beta) V - diag(beta e^gamma) K S0.

Everything is float64. Exponents are only formed for s <= r (differences
<= 0), never e^{-gamma}, so strong decay cannot overflow.
"""
import numpy as np

__all__ = ["gdn_chunked", "chunk_terms"]


def chunk_terms(K, V, g, beta):
    """Per-chunk quantities that do not depend on the state.

    K [C,Dk], V [C,Dv], g [C], beta [C] (float64). Returns a dict with
    gamma, A, T, W, Ut (U~), decay masks.
    """
    C = K.shape[0]
    gamma = np.cumsum(g)
    diff = gamma[:, None] - gamma[None, :]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    lower_strict = np.tril(np.ones((C, C), dtype=bool), -1)
    M_incl = np.exp(np.where(lower_incl, diff, -np.inf))
    M_strict = np.exp(np.where(lower_strict, diff, -np.inf))
    A = beta[:, None] * (K @ K.T) * M_strict
    T = np.linalg.solve(np.eye(C) + A, np.eye(C))
    eg = np.exp(gamma)
    W = T @ ((beta * eg)[:, None] * K)
    Ut = T @ (beta[:, None] * V)
    return {"gamma": gamma, "A": A, "T": T, "W": W, "Ut": Ut,
            "M_incl": M_incl, "eg": eg}


def gdn_chunked(q, k, v, g_log, beta, scale, state=None, chunk=64):
    """Chunked WY form; same contract as :func:`oracle.gdn_serial`.

    Any sequence length is accepted: the last chunk may be shorter.
    Returns (out float64 [B,Hv,S,Dv], state float64 [B,Hv,Dk,Dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g_log = np.asarray(g_log, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    G = Hv // Hk
    out = np.zeros((B, Hv, S, Dv))
    st = np.zeros((B, Hv, Dk, Dv)) if state is None else np.array(state, dtype=np.float64)
    for b in range(B):
        for h in range(Hv):
            j = h // G
            Sc = st[b, h]
            for c0 in range(0, S, chunk):
                c1 = min(S, c0 + chunk)
                K = k[b, j, c0:c1]
                Q = q[b, j, c0:c1]
                V = v[b, h, c0:c1]
                t = chunk_terms(K, V, g_log[b, h, c0:c1], beta[b, h, c0:c1])
                U = t["Ut"] - t["W"] @ Sc
                P = (Q @ K.T) * t["M_incl"]
                out[b, h, c0:c1] = scale * (t["eg"][:, None] * (Q @ Sc) + P @ U)
                gC = t["gamma"][-1]
                Sc = np.exp(gC) * Sc + (np.exp(gC - t["gamma"])[:, None] * K).T @ U
            st[b, h] = Sc
    return out, st

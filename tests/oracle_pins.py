"""Pins for the CPU oracle: facts fixed by the mathematics of the gated delta
rule, independent of the oracle's own code.

Every ``pin_*`` takes an oracle function ``fn(q, k, v, g_log, beta, scale,
state) -> (out, state)`` and raises AssertionError when ``fn`` disagrees.
``test_oracle.py`` runs them on the real oracle (all must hold);
``test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle's C source (each copy must fail at least one).

The recurrence (standard gated delta rule, named by the "GDN CTE Kernel API
Reference" page, introduction and Background):
    S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T
    o_t = scale S_t^T q_t,   value head h reads key head h // (Hv/Hk).
"""
import json
import os

import numpy as np

from oracle.chunked import gdn_chunked

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, B=1, Hk=1, Hv=1, S=8, Dk=4, Dv=3, decay=0.3, state=True):
    """Small random float32 inputs (normalised q, k; beta in (0,1); g < 0)."""
    r = _rng(seed)
    q = _unit(r.standard_normal((B, Hk, S, Dk))).astype(np.float32)
    k = _unit(r.standard_normal((B, Hk, S, Dk))).astype(np.float32)
    v = r.standard_normal((B, Hv, S, Dv)).astype(np.float32)
    g = (-decay * r.uniform(0.1, 2.0, (B, Hv, S))).astype(np.float32)
    beta = r.uniform(0.05, 0.95, (B, Hv, S)).astype(np.float32)
    s0 = (0.5 * r.standard_normal((B, Hv, Dk, Dv))).astype(np.float32) if state else None
    return q, k, v, g, beta, s0


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * ref, "%s: max err %.3e > %.1e" % (what, err, tol * ref)


# ---------------------------------------------------------------- closed forms

def pin_beta_zero_pure_decay(fn):
    """beta = 0 removes the write: S_T = e^{sum g} S_0 and
    o_t = scale e^{sum_{tau<=t} g_tau} S_0^T q_t."""
    q, k, v, g, beta, s0 = random_case(1, B=2, Hk=1, Hv=2, S=9, Dk=4, Dv=3)
    beta[:] = 0.0
    scale = 0.7
    out, st = fn(q, k, v, g, beta, scale, s0)
    G = np.cumsum(g.astype(np.float64), axis=-1)
    for b in range(2):
        for h in range(2):
            S0 = s0[b, h].astype(np.float64)
            for t in range(9):
                exp_o = scale * np.exp(G[b, h, t]) * (S0.T @ q[b, 0, t].astype(np.float64))
                _close(out[b, h, t], exp_o, 1e-12, "beta0 out")
            _close(st[b, h], np.exp(G[b, h, -1]) * S0, 1e-12, "beta0 state")


def pin_orthonormal_overwrite(fn):
    """g = 0, beta = 1, S_0 = 0 and orthonormal keys: every write stores its
    value exactly, S_n = sum_i k_i v_i^T, so S_n^T k_j = v_j; writing an
    already-stored key again replaces its value (S^T k = new v)."""
    r = _rng(2)
    D, Dv = 6, 5
    Qm, _ = np.linalg.qr(r.standard_normal((D, D)))
    keys = Qm.T                                   # rows orthonormal
    k = keys[None, None].astype(np.float32)       # S = D tokens
    kd = k.astype(np.float64)[0, 0]
    q = k.copy()                                  # read back with the keys themselves
    v = r.standard_normal((1, 1, D, Dv)).astype(np.float32)
    g = np.zeros((1, 1, D), np.float32)
    beta = np.ones((1, 1, D), np.float32)
    out, st = fn(q, k, v, g, beta, 1.0, None)
    S_exp = sum(np.outer(kd[i], v[0, 0, i].astype(np.float64)) for i in range(D))
    _close(st[0, 0], S_exp, 1e-6, "orthonormal state")
    _close(st[0, 0].T @ kd.T, v[0, 0].T.astype(np.float64), 1e-6, "orthonormal recall")
    # out_t = S_t^T k_t = v_t (the key just written is read back)
    _close(out[0, 0], v[0, 0], 1e-6, "orthonormal out")
    # overwrite: key 0 written twice, second time with a new value
    k2 = np.concatenate([k, k[:, :, :1]], axis=2)
    v_new = r.standard_normal((1, 1, 1, Dv)).astype(np.float32)
    v2 = np.concatenate([v, v_new], axis=2)
    g2 = np.zeros((1, 1, D + 1), np.float32)
    b2 = np.ones((1, 1, D + 1), np.float32)
    out2, st2 = fn(k2, k2, v2, g2, b2, 1.0, None)
    _close(st2[0, 0].T @ kd[0], v_new[0, 0, 0], 1e-6, "overwrite recall")
    _close(st2[0, 0].T @ kd[1], v[0, 0, 1], 1e-6, "other key untouched")


def pin_single_token_projection(fn):
    """One token, g = 0, beta = 1: S_1 = (I - k k^T) S_0 + k v^T."""
    q, k, v, g, beta, s0 = random_case(3, S=1, Dk=5, Dv=3)
    g[:] = 0.0
    beta[:] = 1.0
    out, st = fn(q, k, v, g, beta, 1.3, s0)
    kk = k[0, 0, 0].astype(np.float64)
    S1 = (np.eye(5) - np.outer(kk, kk)) @ s0[0, 0].astype(np.float64) \
        + np.outer(kk, v[0, 0, 0].astype(np.float64))
    _close(st[0, 0], S1, 1e-12, "projection state")
    _close(out[0, 0, 0], 1.3 * S1.T @ q[0, 0, 0].astype(np.float64), 1e-12, "projection out")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_golden_scalar(fn):
    """Hand-worked Dk = Dv = 1 example (tests/golden/scalar_gdn.json)."""
    d = _golden("scalar_gdn.json")
    n = len(d["g_log"])
    sh = lambda x: np.asarray(x, np.float32).reshape(1, 1, n, 1)
    out, st = fn(sh(d["q"]), sh(d["k"]), sh(d["v"]),
                 np.asarray(d["g_log"], np.float32).reshape(1, 1, n),
                 np.asarray(d["beta"], np.float32).reshape(1, 1, n), d["scale"],
                 np.full((1, 1, 1, 1), d["state0"], np.float32))
    # g_log is stored as float32, so e^{g} is exact to ~1e-7 relative only
    _close(out.reshape(n), d["out"], 1e-6, "golden scalar out")
    _close(st.reshape(()), d["state"], 1e-6, "golden scalar state")


def pin_golden_matrix(fn):
    """Hand-worked Dk = Dv = 2 example with a non-zero start state."""
    d = _golden("matrix_gdn.json")
    n = len(d["g_log"])
    out, st = fn(np.asarray(d["q"], np.float32).reshape(1, 1, n, 2),
                 np.asarray(d["k"], np.float32).reshape(1, 1, n, 2),
                 np.asarray(d["v"], np.float32).reshape(1, 1, n, 2),
                 np.asarray(d["g_log"], np.float32).reshape(1, 1, n),
                 np.asarray(d["beta"], np.float32).reshape(1, 1, n), d["scale"],
                 np.asarray(d["state0"], np.float32).reshape(1, 1, 2, 2))
    _close(out.reshape(n, 2), d["out"], 1e-6, "golden matrix out")
    _close(st.reshape(2, 2), d["state"], 1e-6, "golden matrix state")


# ------------------------------------------------------------- brute force

def pin_bruteforce_products(fn):
    """Explicit Dk x Dk transition products, a different association order:
    Phi_t = e^{g_t} (I - beta_t k_t k_t^T);
    S_t = (Phi_t ... Phi_1) S_0 + sum_{s<=t} (Phi_t ... Phi_{s+1}) beta_s k_s v_s^T;
    o_t = scale S_t^T q_t. GQA with Hk = 2, Hv = 4 (contiguous groups), Dk != Dv."""
    B, Hk, Hv, S, Dk, Dv = 2, 2, 4, 7, 5, 3
    q, k, v, g, beta, s0 = random_case(4, B, Hk, Hv, S, Dk, Dv)
    scale = 0.6
    out, st = fn(q, k, v, g, beta, scale, s0)
    f = lambda x: x.astype(np.float64)
    for b in range(B):
        for h in range(Hv):
            j = h // (Hv // Hk)
            Phi = [np.exp(f(g[b, h, t])) * (np.eye(Dk) - f(beta[b, h, t]) *
                                            np.outer(f(k[b, j, t]), f(k[b, j, t])))
                   for t in range(S)]
            for t in range(S):
                prod_all = np.eye(Dk)
                for s in range(t + 1):
                    prod_all = Phi[s] @ prod_all
                St = prod_all @ f(s0[b, h])
                for s in range(t + 1):
                    tail = np.eye(Dk)
                    for r in range(s + 1, t + 1):
                        tail = Phi[r] @ tail
                    St = St + tail @ (f(beta[b, h, s]) * np.outer(f(k[b, j, s]), f(v[b, h, s])))
                _close(out[b, h, t], scale * St.T @ f(q[b, j, t]), 1e-11, "brute out")
            _close(st[b, h], St, 1e-11, "brute state")


def pin_chunked_agrees(fn):
    """The chunk-parallel WY form (an independent derivation) agrees with the
    token-serial result for chunk sizes 1, 2, 16 and 64, with GQA, ragged
    last chunks and a carried state."""
    for seed, (B, Hk, Hv, S, Dk, Dv), decay in (
            (5, (1, 2, 4, 70, 8, 6), 0.3),
            (6, (2, 1, 2, 131, 16, 12), 0.02),
            (7, (1, 2, 2, 64, 4, 4), 2.0)):
        q, k, v, g, beta, s0 = random_case(seed, B, Hk, Hv, S, Dk, Dv, decay=decay)
        out, st = fn(q, k, v, g, beta, 0.35, s0)
        for C in (1, 2, 16, 64):
            oc, sc = gdn_chunked(q, k, v, g, beta, 0.35, s0, chunk=C)
            _close(out, oc, 1e-10, "chunked out C=%d" % C)
            _close(st, sc, 1e-10, "chunked state C=%d" % C)


# --------------------------------------------------------------- invariants

def pin_gqa_equals_repeat(fn):
    """GQA (Hv = G * Hk) equals running with q, k explicitly repeated per
    value head in contiguous groups (value head h uses key head h // G)."""
    q, k, v, g, beta, s0 = random_case(8, B=2, Hk=2, Hv=6, S=11, Dk=4, Dv=5)
    o1, s1 = fn(q, k, v, g, beta, 0.5, s0)
    qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
    o2, s2 = fn(qr, kr, v, g, beta, 0.5, s0)
    _close(o1, o2, 1e-13, "gqa out")
    _close(s1, s2, 1e-13, "gqa state")


def pin_columns_independent(fn):
    """Each value column evolves on its own: running Dv columns together equals
    running each column alone (Dv = 1)."""
    q, k, v, g, beta, s0 = random_case(9, B=1, Hk=1, Hv=2, S=13, Dk=5, Dv=4)
    o, s = fn(q, k, v, g, beta, 1.0, s0)
    for c in range(4):
        oc, sc = fn(q, k, v[..., c:c + 1].copy(), g, beta, 1.0, s0[..., c:c + 1].copy())
        _close(o[..., c:c + 1], oc, 1e-13, "column out")
        _close(s[..., c:c + 1], sc, 1e-13, "column state")


def pin_linear_in_values_and_state(fn):
    """For fixed q, k, g, beta the map (V, S_0) -> (out, S_T) is linear."""
    q, k, v, g, beta, s0 = random_case(10, B=1, Hk=1, Hv=1, S=12, Dk=4, Dv=3)
    _, _, v2, _, _, s02 = random_case(11, B=1, Hk=1, Hv=1, S=12, Dk=4, Dv=3)
    a, c = 0.75, -1.5
    o1, t1 = fn(q, k, v, g, beta, 1.0, s0)
    o2, t2 = fn(q, k, v2, g, beta, 1.0, s02)
    o3, t3 = fn(q, k, (a * v + c * v2).astype(np.float32), g, beta, 1.0,
                (a * s0 + c * s02).astype(np.float32))
    # float32 rounding of the combined inputs bounds the agreement
    _close(o3, a * o1 + c * o2, 1e-6, "linear out")
    _close(t3, a * t1 + c * t2, 1e-6, "linear state")


def pin_scale(fn):
    """out is linear in scale; the state does not depend on it."""
    q, k, v, g, beta, s0 = random_case(12, S=10)
    o1, t1 = fn(q, k, v, g, beta, 1.0, s0)
    o2, t2 = fn(q, k, v, g, beta, 0.125, s0)
    _close(o2, 0.125 * o1, 1e-14, "scale out")
    _close(t2, t1, 0.0, "scale state")


def pin_split_carry(fn):
    """Running S1 tokens, then S2 tokens from the carried state, equals
    running S1 + S2 tokens at once (the state is the resume point)."""
    q, k, v, g, beta, s0 = random_case(13, B=1, Hk=1, Hv=2, S=20, Dk=4, Dv=3)
    o, s = fn(q, k, v, g, beta, 0.9, s0)
    cut = 7
    oa, sa = fn(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], g[..., :cut], beta[..., :cut],
                0.9, s0)
    ob, sb = fn(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], g[..., cut:], beta[..., cut:],
                0.9, sa)
    _close(np.concatenate([oa, ob], axis=2), o, 1e-6, "split out")
    _close(sb, s, 1e-6, "split state")


def pin_permutation(fn):
    """Permuting batches permutes results; permuting value heads inside a GQA
    group (which share q, k) permutes results."""
    q, k, v, g, beta, s0 = random_case(14, B=3, Hk=1, Hv=3, S=6, Dk=4, Dv=3)
    o, s = fn(q, k, v, g, beta, 1.0, s0)
    pb, ph = [2, 0, 1], [1, 2, 0]
    o2, s2 = fn(q[pb], k[pb], v[pb][:, ph], g[pb][:, ph], beta[pb][:, ph], 1.0, s0[pb][:, ph])
    _close(o2, o[pb][:, ph], 1e-14, "perm out")
    _close(s2, s[pb][:, ph], 1e-14, "perm state")


ALL_PINS = [
    pin_beta_zero_pure_decay, pin_orthonormal_overwrite, pin_single_token_projection,
    pin_golden_scalar, pin_golden_matrix, pin_bruteforce_products, pin_chunked_agrees,
    pin_gqa_equals_repeat, pin_columns_independent, pin_linear_in_values_and_state,
    pin_scale, pin_split_carry, pin_permutation,
]


# ------------------------------------------------- gate + normalisation prologue
#
# The decode block computes the recurrence's inputs from raw quantities
# ("GDN Block TKG Kernel API Reference": introduction, "l2norm/beta/g";
# Parameters A_log, a per-value-head log decay, and dt_bias, a per-value-head
# softplus bias); q and k must reach the recurrence L2-normalised ("GDN CTE
# Kernel API Reference", Notes). Read here as, per token,
#     g_log = -exp(A_log[h]) softplus(a + dt_bias[h]),  beta = sigmoid(b),
#     k = k_raw / sqrt(|k_raw|^2 + eps), q likewise.
# Every ``gpin_*`` takes a namespace ``o`` with
#     o.gated(q, k, v, a, b, A_log, dt_bias, scale, eps, state) -> (out, state)
#     o.gates(a, b, A_log, dt_bias) -> (g_log, beta)
#     o.l2norm(x, eps) -> x normalised over its last axis
# and checks them against library routines (scipy's logistic function),
# closed forms and a hand-worked example.

def _expit(x):
    from scipy.special import expit
    return expit(np.asarray(x, np.float64))


def raw_case(seed, B=1, Hk=1, Hv=1, S=8, Dk=4, Dv=3, state=True):
    """Small random raw prologue inputs: un-normalised q, k (norms spread over
    [0.2, 5]), v, gate pre-activations a, b and per-head A_log, dt_bias."""
    r = _rng(seed)
    q = (r.standard_normal((B, Hk, S, Dk)) * r.uniform(0.2, 5.0, (B, Hk, S, 1))).astype(np.float32)
    k = (r.standard_normal((B, Hk, S, Dk)) * r.uniform(0.2, 5.0, (B, Hk, S, 1))).astype(np.float32)
    v = r.standard_normal((B, Hv, S, Dv)).astype(np.float32)
    a = r.standard_normal((B, Hv, S)).astype(np.float32)
    b = r.standard_normal((B, Hv, S)).astype(np.float32)
    A_log = r.uniform(np.log(1.0), np.log(16.0), Hv).astype(np.float32)
    dt_bias = r.uniform(-1.0, 1.0, Hv).astype(np.float32)
    s0 = (0.5 * r.standard_normal((B, Hv, Dk, Dv))).astype(np.float32) if state else None
    return q, k, v, a, b, A_log, dt_bias, s0


def _decay_by_library(a, A_log, dt_bias):
    """e^{g} = exp(-e^{A} softplus(x)) = (1 / (1 + e^{x}))^{e^{A}} = expit(-x)^{e^{A}}."""
    x = a.astype(np.float64) + dt_bias.astype(np.float64)[None, :, None]
    return _expit(-x) ** np.exp(A_log.astype(np.float64))[None, :, None]


def gpin_gates_match_library(o):
    """e^{g} equals expit(-(a + dt_bias))^{exp(A_log)} and beta equals expit(b),
    with A_log and dt_bias varying per value head; extreme pre-activations stay
    finite and follow the asymptotes of softplus."""
    _, _, _, a, b, A_log, dt_bias, _ = raw_case(30, B=2, Hv=3, S=7)
    g, beta = o.gates(a, b, A_log, dt_bias)
    _close(np.exp(g), _decay_by_library(a, A_log, dt_bias), 1e-12, "gates: decay")
    _close(beta, _expit(b), 1e-14, "gates: beta")
    assert np.all(g < 0), "gates: g_log must be negative"
    # asymptotes: softplus(x) -> x for large x, -> e^x for very negative x
    a2 = np.array([[[60.0, -60.0, 0.0]]], np.float32)
    b2 = np.array([[[60.0, -60.0, 0.0]]], np.float32)
    g2, be2 = o.gates(a2, b2, np.array([np.log(2.0)], np.float32), np.zeros(1, np.float32))
    e2 = np.exp(float(np.float32(np.log(2.0))))
    assert np.all(np.isfinite(g2)) and np.all(np.isfinite(be2)), "gates: not finite"
    _close(g2[0, 0, 0] / (-e2 * 60.0), 1.0, 1e-14, "gates: large x")
    _close(g2[0, 0, 1] / (-e2 * np.exp(-60.0)), 1.0, 1e-12, "gates: small x")
    _close(g2[0, 0, 2], -e2 * np.log(2.0), 1e-15, "gates: x = 0")
    _close(be2[0, 0], [1.0, np.exp(-60.0), 0.5], 1e-15, "gates: beta limits")


def gpin_l2norm_closed_forms(o):
    """(3, 4) -> (0.6, 0.8); with eps = 11 the divisor is sqrt(25 + 11) = 6;
    a zero vector stays zero; random rows get unit norm and keep direction."""
    _close(o.l2norm(np.array([[3.0, 4.0]], np.float32), 0.0), [[0.6, 0.8]], 1e-15, "l2 (3,4)")
    _close(o.l2norm(np.array([[3.0, 4.0]], np.float32), 11.0), [[0.5, 4.0 / 6.0]], 1e-15,
           "l2 eps")
    z = o.l2norm(np.zeros((2, 5), np.float32), 1e-6)
    assert np.all(z == 0.0), "l2: zero vector"
    x = _rng(31).standard_normal((3, 4, 7)).astype(np.float32) * 3.0
    y = o.l2norm(x, 0.0)
    _close(np.linalg.norm(y, axis=-1), np.ones((3, 4)), 1e-14, "l2: unit norm")
    _close(y * np.linalg.norm(x.astype(np.float64), axis=-1, keepdims=True),
           x.astype(np.float64), 1e-13, "l2: direction")


def gpin_gated_golden(o):
    """Hand-worked Dk = 2 example (tests/golden/gated_gdn.json)."""
    d = _golden("gated_gdn.json")
    n = len(d["v"])
    f = lambda x, *s: np.asarray(x, np.float32).reshape(*s)
    out, st = o.gated(f(d["q"], 1, 1, n, 2), f(d["k"], 1, 1, n, 2), f(d["v"], 1, 1, n, 1),
                      f(d["a"], 1, 1, n), f(d["b"], 1, 1, n), f([d["A_log"]], 1),
                      f([d["dt_bias"]], 1), d["scale"], d["eps"], f(d["state0"], 1, 1, 2, 1))
    # the logarithms are stored as float32: e^{g} is exact to ~1e-7 relative
    _close(out.reshape(n), d["out"], 1e-6, "gated golden out")
    _close(st.reshape(2), d["state"], 1e-6, "gated golden state")


def gpin_gated_pure_decay(o):
    """b = -60 makes beta ~ 1e-26: no write, S_T = prod e^{g_t} S_0 and
    o_t = scale (prod_{tau<=t} e^{g_tau}) S_0^T q_t / |q_t|, with e^{g} from the
    logistic function (library)."""
    q, k, v, a, b, A_log, dt_bias, s0 = raw_case(32, B=1, Hk=1, Hv=2, S=6, Dk=4, Dv=3)
    b[:] = -60.0
    out, st = o.gated(q, k, v, a, b, A_log, dt_bias, 0.8, 0.0, s0)
    dec = np.cumprod(_decay_by_library(a, A_log, dt_bias), axis=-1)
    qn = q.astype(np.float64) / np.linalg.norm(q.astype(np.float64), axis=-1, keepdims=True)
    for h in range(2):
        S0 = s0[0, h].astype(np.float64)
        for t in range(6):
            _close(out[0, h, t], 0.8 * dec[0, h, t] * (S0.T @ qn[0, 0, t]), 1e-12, "decay out")
        _close(st[0, h], dec[0, h, -1] * S0, 1e-12, "decay state")


def gpin_gated_equals_normalised_serial(o):
    """The prologue followed by the recurrence equals the (separately pinned)
    serial recurrence fed with q, k normalised by numpy and g_log, beta from
    the logistic function, with GQA (Hk = 2, Hv = 4) and per-head parameters."""
    import oracle
    q, k, v, a, b, A_log, dt_bias, s0 = raw_case(33, B=2, Hk=2, Hv=4, S=9, Dk=5, Dv=3)
    eps = 1e-3
    out, st = o.gated(q, k, v, a, b, A_log, dt_bias, 0.6, eps, s0)
    nq = lambda x: x.astype(np.float64) / np.sqrt(
        np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True) + eps)
    g = np.log(_decay_by_library(a, A_log, dt_bias))
    ref_o, ref_s = oracle.gdn_serial(nq(q), nq(k), v, g, _expit(b), 0.6, s0)
    # the serial oracle takes float32 inputs: agreement to float32 rounding
    _close(out, ref_o, 2e-6, "gated vs serial out")
    _close(st, ref_s, 2e-6, "gated vs serial state")


def gpin_gated_norm_invariance(o):
    """With eps = 0 the result does not depend on the length of each q_t and
    k_t: rescaling every token's q and k by its own positive factor changes
    nothing."""
    q, k, v, a, b, A_log, dt_bias, s0 = raw_case(34, B=1, Hk=1, Hv=2, S=10, Dk=6, Dv=4)
    o1, s1 = o.gated(q, k, v, a, b, A_log, dt_bias, 1.1, 0.0, s0)
    r = _rng(35)
    # powers of two keep the rescaled float32 inputs exact
    fq = (2.0 ** r.integers(-4, 5, (1, 1, 10, 1))).astype(np.float32)
    fk = (2.0 ** r.integers(-4, 5, (1, 1, 10, 1))).astype(np.float32)
    o2, s2 = o.gated(q * fq, k * fk, v, a, b, A_log, dt_bias, 1.1, 0.0, s0)
    _close(o2, o1, 1e-13, "norm invariance out")
    _close(s2, s1, 1e-13, "norm invariance state")


def gpin_gated_heads_independent(o):
    """Each value head uses its own A_log[h], dt_bias[h]: a GQA call equals
    one single-head call per value head (with that head's key head)."""
    q, k, v, a, b, A_log, dt_bias, s0 = raw_case(36, B=1, Hk=2, Hv=4, S=7, Dk=4, Dv=3)
    out, st = o.gated(q, k, v, a, b, A_log, dt_bias, 0.9, 1e-6, s0)
    for h in range(4):
        j = h // 2
        sl = slice(h, h + 1)
        oh, sh = o.gated(q[:, j:j + 1], k[:, j:j + 1], v[:, sl], a[:, sl], b[:, sl],
                         A_log[sl], dt_bias[sl], 0.9, 1e-6, s0[:, sl])
        _close(out[:, sl], oh, 1e-14, "heads out")
        _close(st[:, sl], sh, 1e-14, "heads state")


def gpin_gated_f64_inputs(o):
    """The fp64-input entry gives exactly the float entry's result on inputs
    that float32 represents exactly, and differs on inputs it does not."""
    q, k, v, a, b, A_log, dt_bias, s0 = raw_case(37, B=1, Hk=1, Hv=2, S=6, Dk=4, Dv=3)
    o1, s1 = o.gated(q, k, v, a, b, A_log, dt_bias, 0.7, 1e-6, s0)
    f = lambda x: x.astype(np.float64)
    o2, s2 = o.gated_f64(f(q), f(k), f(v), f(a), f(b), f(A_log), f(dt_bias), 0.7, 1e-6, s0)
    _close(o2, o1, 0.0, "f64 entry out")
    _close(s2, s1, 0.0, "f64 entry state")
    v3 = f(v) + 1e-9                                  # not representable in float32
    o3, _ = o.gated_f64(f(q), f(k), v3, f(a), f(b), f(A_log), f(dt_bias), 0.7, 1e-6, s0)
    assert np.max(np.abs(o3 - o1)) > 0.0, "f64 entry must read double inputs"


GATED_PINS = [
    gpin_gates_match_library, gpin_l2norm_closed_forms, gpin_gated_golden,
    gpin_gated_pure_decay, gpin_gated_equals_normalised_serial, gpin_gated_norm_invariance,
    gpin_gated_heads_independent, gpin_gated_f64_inputs,
]


# --------------------------------------------------- depthwise causal conv1d
#
# "GDN Conv1D Kernel API Reference": prefill returns silu(causal depthwise
# conv1d(mixed)) and the last K raw tokens; decode shifts the window by the
# new token and returns silu of the K-tap dot product. Every ``cpin_*`` takes
# a namespace ``o`` with o.prefill(x, w) -> (out, state) and
# o.decode(x, state, w) -> (out, new_state), checked against library filters
# (scipy.signal.lfilter, numpy.convolve), the logistic function, an impulse
# response and the prefill/decode chain.

def conv_case(seed, B=2, C=5, T=11, K=4):
    r = _rng(seed)
    x = r.standard_normal((B, C, T)).astype(np.float32)
    w = (r.standard_normal((C, K)) * 0.5).astype(np.float32)
    return x, w


def cpin_matches_lfilter(o):
    """Per channel, the pre-activation is the FIR y[n] = sum_k b[k] x[n-k] with
    b = the weights reversed (scipy.signal.lfilter), and out = y * expit(y)."""
    from scipy.signal import lfilter
    x, w = conv_case(40, B=2, C=3, T=13, K=4)
    out, _ = o.prefill(x, w)
    for b in range(2):
        for c in range(3):
            y = lfilter(w[c, ::-1].astype(np.float64), [1.0], x[b, c].astype(np.float64))
            _close(out[b, c], y * _expit(y), 1e-13, "conv vs lfilter")


def cpin_matches_convolve(o):
    """The same through numpy.convolve (full convolution, first T outputs),
    for every K from 1 to 8 and T shorter and longer than K."""
    for K in range(1, 9):
        for T in (1, K - 1, K, 3 * K + 2):
            if T < 1:
                continue
            x, w = conv_case(41 + K, B=1, C=2, T=T, K=K)
            out, _ = o.prefill(x, w)
            for c in range(2):
                y = np.convolve(x[0, c].astype(np.float64), w[c].astype(np.float64)[::-1])[:T]
                _close(out[0, c], y * _expit(y), 1e-13, "conv vs convolve K=%d T=%d" % (K, T))


def cpin_impulse_response(o):
    """A unit impulse at t0 gives pre-activations w[K-1], w[K-2], ..., w[0] at
    t0, t0+1, ..., t0+K-1 (the current token takes the last weight) and zero
    elsewhere; silu maps them through y / (1 + e^{-y})."""
    K, T, t0 = 4, 12, 3
    x = np.zeros((1, 1, T), np.float32)
    x[0, 0, t0] = 1.0
    w = np.array([[0.5, -1.0, 2.0, 3.0]], np.float32)
    out, _ = o.prefill(x, w)
    y = np.zeros(T)
    y[t0:t0 + K] = [3.0, 2.0, -1.0, 0.5]
    _close(out[0, 0], y / (1.0 + np.exp(-y)), 1e-15, "impulse")
    # silu closed forms: silu(0) = 0, silu(3) = 3 / (1 + e^-3)
    assert out[0, 0, 0] == 0.0 and out[0, 0, T - 1] == 0.0


def cpin_state_is_last_raw_tokens(o):
    """The prefill state is the last K raw (pre-convolution) tokens, with
    zeros in front when T < K."""
    x, w = conv_case(50, B=2, C=3, T=9, K=4)
    _, st = o.prefill(x, w)
    _close(st, x[:, :, 5:9], 0.0, "state = last K raw")
    x2, w2 = conv_case(51, B=1, C=2, T=2, K=4)
    _, st2 = o.prefill(x2, w2)
    exp = np.zeros((1, 2, 4))
    exp[:, :, 2:] = x2
    _close(st2, exp, 0.0, "state with T < K")


def cpin_decode_continues_prefill(o):
    """prefill(T) followed by n decode steps equals prefill(T + n): outputs
    and window state, for K = 3 and K = 4."""
    for K in (3, 4):
        x, w = conv_case(52 + K, B=2, C=4, T=10, K=K)
        full_out, full_st = o.prefill(x, w)
        out, st = o.prefill(x[:, :, :6], w)
        _close(out, full_out[:, :, :6], 1e-15, "prefix")
        for t in range(6, 10):
            ot, st = o.decode(x[:, :, t], st, w)
            _close(ot, full_out[:, :, t], 1e-13, "decode step t=%d K=%d" % (t, K))
        _close(st, full_st, 0.0, "decode window state")


def cpin_decode_window_shift(o):
    """A decode step drops the oldest token and appends the new one, and its
    output is silu(sum_j w_j window_j), worked by hand for K = 3."""
    st = np.array([[[1.0, 2.0, 3.0]]], np.float32)
    w = np.array([[0.5, -1.0, 0.25]], np.float32)
    out, nst = o.decode(np.array([[4.0]], np.float32), st, w)
    _close(nst, [[[2.0, 3.0, 4.0]]], 0.0, "window shift")
    y = 0.5 * 2.0 - 1.0 * 3.0 + 0.25 * 4.0          # = -1
    _close(out, [[y / (1.0 + np.exp(-y))]], 1e-15, "decode dot product")


def cpin_channels_independent(o):
    """Each channel uses only its own weights and its own input row."""
    x, w = conv_case(56, B=1, C=4, T=9, K=3)
    out, st = o.prefill(x, w)
    for c in range(4):
        oc, sc = o.prefill(x[:, c:c + 1], w[c:c + 1])
        _close(out[:, c:c + 1], oc, 0.0, "channel out")
        _close(st[:, c:c + 1], sc, 0.0, "channel state")


CONV_PINS = [
    cpin_matches_lfilter, cpin_matches_convolve, cpin_impulse_response,
    cpin_state_is_last_raw_tokens, cpin_decode_continues_prefill, cpin_decode_window_shift,
    cpin_channels_independent,
]


# ------------------------------------------- RMSNormGated and the decode block
#
# RMSNormGated ("GDN Block TKG Kernel API Reference": introduction, norm_weight
# gamma over head_v_dim, gated by the z projection), read as
#     y = o / sqrt(mean(o^2) + eps) * gamma * silu(z)   over each head's Dv.
# ``rpin_*`` take a namespace with o.rmsnorm(o, z, w, eps) and
# o.block(...) (oracle.block.decode_block's signature).

def rpin_rmsnorm_matches_torch(o):
    """Against torch.nn.functional.rms_norm and silu in float64."""
    import torch
    import torch.nn.functional as F
    r = _rng(60)
    x = r.standard_normal((3, 4, 16)) * 2.0
    z = r.standard_normal((3, 4, 16)) * 3.0
    w = r.uniform(0.5, 1.5, 16)
    for eps in (0.0, 1e-6, 0.3):
        y = o.rmsnorm(x, z, w, eps)
        t = F.rms_norm(torch.from_numpy(x), (16,), weight=torch.from_numpy(w), eps=eps) \
            * F.silu(torch.from_numpy(z))
        _close(y, t.numpy(), 1e-13, "rmsnorm vs torch eps=%g" % eps)


def rpin_rmsnorm_closed_forms(o):
    """A constant row c gives c / sqrt(c^2 + eps); z = 0 gives 0; with eps = 0
    scaling o changes nothing."""
    D = 8
    y = o.rmsnorm(np.full((1, D), 3.0), np.full((1, D), 50.0), np.ones(D), 16.0)
    _close(y, np.full((1, D), 3.0 / 5.0 * 50.0), 1e-13, "constant row")   # silu(50) = 50
    y0 = o.rmsnorm(_rng(61).standard_normal((2, D)), np.zeros((2, D)), np.ones(D), 1e-6)
    assert np.all(y0 == 0.0), "silu(0) = 0 gates everything off"
    x = _rng(62).standard_normal((2, 3, D))
    z = _rng(63).standard_normal((2, 3, D))
    w = _rng(64).uniform(0.5, 2.0, D)
    _close(o.rmsnorm(7.5 * x, z, w, 0.0), o.rmsnorm(x, z, w, 0.0), 1e-14, "scale invariance")


def block_case(seed, B=2, Hk=2, Hv=4, Dk=4, Dv=3, K=4):
    r = _rng(seed)
    C = 2 * Hk * Dk + Hv * Dv
    return dict(
        mixed=r.standard_normal((B, C)).astype(np.float32),
        z=r.standard_normal((B, Hv * Dv)).astype(np.float32),
        a=r.standard_normal((B, Hv)).astype(np.float32),
        b=r.standard_normal((B, Hv)).astype(np.float32),
        conv_state=r.standard_normal((B, C, K)).astype(np.float32),
        conv_weight=(r.uniform(-1, 1, (C, K)) / np.sqrt(K)).astype(np.float32),
        A_log=r.uniform(0.0, np.log(16.0), Hv).astype(np.float32),
        dt_bias=r.uniform(-1, 1, Hv).astype(np.float32),
        norm_weight=r.uniform(0.5, 1.5, Dv).astype(np.float32),
        state=(0.5 * r.standard_normal((B, Hv, Dk, Dv))).astype(np.float32),
        scale=0.5, l2_eps=1e-6, norm_eps=1e-5, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv)


def bpin_block_from_library_steps(o):
    """The block equals its steps done with library routines: the conv window
    as an explicit dot product and scipy's logistic function, the q|k|v split
    in that channel order, numpy norms, gates from the logistic function, the
    (separately pinned) token-serial recurrence on those inputs, and torch's
    rms_norm times silu(z)."""
    import oracle
    import torch
    import torch.nn.functional as F
    d = block_case(65)
    B, Hk, Hv, Dk, Dv = 2, d["Hk"], d["Hv"], d["Dk"], d["Dv"]
    out, conv_st, st = o.block(**d)
    f = lambda x: np.asarray(x, np.float64)
    win = np.concatenate([f(d["conv_state"])[:, :, 1:], f(d["mixed"])[:, :, None]], axis=2)
    pre = np.einsum("bck,ck->bc", win, f(d["conv_weight"]))
    xc = pre * _expit(pre)
    _close(conv_st, win, 0.0, "block conv state")
    q = xc[:, :Hk * Dk].reshape(B, Hk, 1, Dk)
    k = xc[:, Hk * Dk:2 * Hk * Dk].reshape(B, Hk, 1, Dk)
    v = xc[:, 2 * Hk * Dk:].reshape(B, Hv, 1, Dv)
    nrm = lambda x: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + d["l2_eps"])
    g = np.log(_decay_by_library(d["a"][:, :, None], d["A_log"], d["dt_bias"]))
    ro, rs = oracle.gdn_serial(nrm(q), nrm(k), v, g, _expit(d["b"])[:, :, None], d["scale"],
                               d["state"])
    _close(st, rs, 2e-6, "block state")         # the serial oracle takes float32 inputs
    zz = torch.from_numpy(f(d["z"]).reshape(B, Hv, Dv))
    y = F.rms_norm(torch.from_numpy(ro[:, :, 0]), (Dv,), weight=torch.from_numpy(f(d["norm_weight"])),
                   eps=d["norm_eps"]) * F.silu(zz)
    _close(out, y.numpy().reshape(B, Hv * Dv), 2e-5, "block out")


def bpin_block_chain_matches_prefill(o):
    """Three block steps from a zero conv window equal one conv prefill of the
    three tokens followed by the gated recurrence over them (the state and
    the normalised outputs of each step)."""
    import oracle
    from oracle import conv1d
    d = block_case(66, B=1, Hk=1, Hv=2, Dk=4, Dv=3, K=3)
    Hk, Hv, Dk, Dv = d["Hk"], d["Hv"], d["Dk"], d["Dv"]
    C = d["mixed"].shape[1]
    r = _rng(67)
    toks = r.standard_normal((3, 1, C)).astype(np.float32)
    zs = r.standard_normal((3, 1, Hv * Dv)).astype(np.float32)
    a3 = r.standard_normal((3, 1, Hv)).astype(np.float32)
    b3 = r.standard_normal((3, 1, Hv)).astype(np.float32)
    cs = np.zeros((1, C, 3), np.float32)
    st = d["state"]
    outs = []
    for t in range(3):
        dd = dict(d, mixed=toks[t], z=zs[t], a=a3[t], b=b3[t], conv_state=cs, state=st)
        y, cs, st = o.block(**dd)
        outs.append(y)
    xc, _ = conv1d.conv1d_prefill(np.transpose(toks, (1, 2, 0)), d["conv_weight"])   # [1, C, 3]
    q = np.transpose(xc[:, :Hk * Dk].reshape(1, Hk, Dk, 3), (0, 1, 3, 2))
    k = np.transpose(xc[:, Hk * Dk:2 * Hk * Dk].reshape(1, Hk, Dk, 3), (0, 1, 3, 2))
    v = np.transpose(xc[:, 2 * Hk * Dk:].reshape(1, Hv, Dv, 3), (0, 1, 3, 2))
    ro, rs = oracle.gdn_serial_gated_f64(q, k, v, np.transpose(a3, (1, 2, 0)),
                                         np.transpose(b3, (1, 2, 0)), d["A_log"], d["dt_bias"],
                                         d["scale"], d["l2_eps"], d["state"])
    _close(st, rs, 1e-12, "chained block state")
    for t in range(3):
        y = o.rmsnorm(ro[:, :, t], zs[t].reshape(1, Hv, Dv), d["norm_weight"], d["norm_eps"])
        _close(outs[t], y.reshape(1, Hv * Dv), 1e-12, "chained block out %d" % t)


RMS_PINS = [rpin_rmsnorm_matches_torch, rpin_rmsnorm_closed_forms,
            bpin_block_from_library_steps, bpin_block_chain_matches_prefill]

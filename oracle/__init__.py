"""CPU oracle for the gated delta-rule recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it and
shares no code with it.

* :func:`gdn_serial` -- the definition: token-serial fp64 recurrence (C, see
  ``gdn_serial.c``), S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T,
  o_t = scale S_t^T q_t, with value head h reading key head h // (Hv/Hk)
  (page "GDN CTE Kernel API Reference", Notes).
* :func:`gdn_serial_gated` -- the same recurrence behind the decode block's
  prologue: g_log = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b),
  q and k L2-normalised with an epsilon (page "GDN Block TKG Kernel API
  Reference", introduction and Parameters A_log, dt_bias).
* :func:`gdn_gates`, :func:`l2_normalize` -- those two prologue steps alone.
* :mod:`oracle.chunked` -- an independent chunk-parallel (WY) derivation in
  numpy fp64, used only as a cross-check of :func:`gdn_serial`.
"""
import ctypes
import os

import numpy as np

from . import build as _build

__all__ = ["gdn_serial", "gdn_serial_gated", "gdn_serial_gated_f64", "gdn_gates", "l2_normalize",
           "default_threads"]

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_gdn_serial.restype = ctypes.c_int
        lib.oracle_gdn_serial.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_long, ctypes.c_int]
        lib.oracle_gdn_serial_gated.restype = ctypes.c_int
        lib.oracle_gdn_serial_gated.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_long, ctypes.c_int]
        lib.oracle_gdn_serial_gated_f64.restype = ctypes.c_int
        lib.oracle_gdn_serial_gated_f64.argtypes = lib.oracle_gdn_serial_gated.argtypes
        lib.oracle_gdn_gates.restype = ctypes.c_int
        lib.oracle_gdn_gates.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_long] * 3
        lib.oracle_l2norm.restype = ctypes.c_int
        lib.oracle_l2norm.argtypes = [ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                      ctypes.c_long, ctypes.c_long]
        _LIB = lib
    return _LIB


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _state_arg(state, shape, inplace):
    if state is None:
        return np.zeros(shape, dtype=np.float64)
    if inplace:
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous and state.shape == shape):
            raise ValueError("oracle: inplace needs a C-contiguous float64 state of the right shape")
        return state
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    if st.shape != shape:
        raise ValueError("oracle: bad state shape")
    return st


def gdn_serial(q, k, v, g_log, beta, scale, state=None, nthreads=None, inplace=False):
    """Token-serial fp64 gated delta rule.

    Shapes: q, k [B,Hk,S,Dk]; v [B,Hv,S,Dv]; g_log, beta [B,Hv,S];
    state [B,Hv,Dk,Dv] or None (zero initial state).
    Inputs are taken as float32 (bf16 values are exact in float32).
    Returns (out [B,Hv,S,Dv] float64, final state [B,Hv,Dk,Dv] float64).
    With ``inplace=True`` a C-contiguous float64 ``state`` is updated in place
    (and returned) instead of copied, for long chains of decode steps.
    """
    q, k, v, g_log, beta = (_f32(a) for a in (q, k, v, g_log, beta))
    B, Hk, S, Dk = q.shape
    Bv, Hv, Sv, Dv = v.shape
    if k.shape != q.shape or (Bv, Sv) != (B, S) or g_log.shape != (B, Hv, S) \
            or beta.shape != (B, Hv, S):
        raise ValueError("oracle: inconsistent shapes")
    if Hv % Hk:
        raise ValueError("oracle: Hv must be a multiple of Hk")
    st = _state_arg(state, (B, Hv, Dk, Dv), inplace)
    out = np.empty((B, Hv, S, Dv), dtype=np.float64)
    n = default_threads() if nthreads is None else int(nthreads)
    rc = _lib().oracle_gdn_serial(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, g_log.ctypes.data, beta.ctypes.data,
        float(scale), st.ctypes.data, out.ctypes.data, B, Hk, Hv, S, Dk, Dv, n)
    if rc != 0:
        raise RuntimeError("oracle_gdn_serial failed with code %d" % rc)
    return out, st


def gdn_serial_gated(q, k, v, a, b, A_log, dt_bias, scale, eps, state=None, nthreads=None,
                     inplace=False, _f64=False):
    """Token-serial fp64 gated delta rule from the raw prologue inputs.

    Shapes: q, k [B,Hk,S,Dk] (not normalised); v [B,Hv,S,Dv]; a, b [B,Hv,S];
    A_log, dt_bias [Hv]; state [B,Hv,Dk,Dv] or None. Per token
    g_log = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b),
    q and k divided by sqrt(sum of squares + eps), all in fp64; then the
    recurrence of :func:`gdn_serial`. Returns (out, final state), float64.
    """
    conv = (lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float64))) if _f64 else _f32
    q, k, v, a, b, A_log, dt_bias = (conv(x) for x in (q, k, v, a, b, A_log, dt_bias))
    B, Hk, S, Dk = q.shape
    Bv, Hv, Sv, Dv = v.shape
    if k.shape != q.shape or (Bv, Sv) != (B, S) or a.shape != (B, Hv, S) \
            or b.shape != (B, Hv, S) or A_log.shape != (Hv,) or dt_bias.shape != (Hv,):
        raise ValueError("oracle: inconsistent shapes")
    if Hv % Hk:
        raise ValueError("oracle: Hv must be a multiple of Hk")
    st = _state_arg(state, (B, Hv, Dk, Dv), inplace)
    out = np.empty((B, Hv, S, Dv), dtype=np.float64)
    n = default_threads() if nthreads is None else int(nthreads)
    fn = _lib().oracle_gdn_serial_gated_f64 if _f64 else _lib().oracle_gdn_serial_gated
    rc = fn(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, a.ctypes.data, b.ctypes.data,
        A_log.ctypes.data, dt_bias.ctypes.data, float(eps), float(scale),
        st.ctypes.data, out.ctypes.data, B, Hk, Hv, S, Dk, Dv, n)
    if rc != 0:
        raise RuntimeError("oracle_gdn_serial_gated failed with code %d" % rc)
    return out, st


def gdn_serial_gated_f64(q, k, v, a, b, A_log, dt_bias, scale, eps, state=None,
                         nthreads=None, inplace=False):
    """:func:`gdn_serial_gated` with every input taken in float64 (for inputs
    that are themselves fp64 results, such as the conv1d output)."""
    return gdn_serial_gated(q, k, v, a, b, A_log, dt_bias, scale, eps, state, nthreads,
                            inplace, _f64=True)


def gdn_gates(a, b, A_log, dt_bias):
    """g_log = -exp(A_log[h]) softplus(a + dt_bias[h]) and beta = sigmoid(b),
    fp64, for a, b [B,Hv,S] and A_log, dt_bias [Hv]."""
    a, b, A_log, dt_bias = (_f32(x) for x in (a, b, A_log, dt_bias))
    if a.ndim != 3 or b.shape != a.shape or A_log.shape != (a.shape[1],) \
            or dt_bias.shape != A_log.shape:
        raise ValueError("oracle: inconsistent gate shapes")
    B, Hv, S = a.shape
    g = np.empty(a.shape, np.float64)
    be = np.empty(a.shape, np.float64)
    rc = _lib().oracle_gdn_gates(a.ctypes.data, b.ctypes.data, A_log.ctypes.data,
                                 dt_bias.ctypes.data, g.ctypes.data, be.ctypes.data, B, Hv, S)
    if rc != 0:
        raise RuntimeError("oracle_gdn_gates failed with code %d" % rc)
    return g, be


def l2_normalize(x, eps):
    """x / sqrt(sum over the last axis of x^2 + eps), fp64."""
    x = _f32(x)
    D = x.shape[-1]
    y = np.empty(x.shape, np.float64)
    rc = _lib().oracle_l2norm(x.ctypes.data, float(eps), y.ctypes.data, x.size // D if D else 0, D)
    if rc != 0:
        raise RuntimeError("oracle_l2norm failed with code %d" % rc)
    return y

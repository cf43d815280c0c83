"""CPU oracle for the gated delta-rule recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it and
shares no code with it.

* :func:`gdn_serial` -- the definition: token-serial fp64 recurrence (C, see
  ``gdn_serial.c``), S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T,
  o_t = scale S_t^T q_t, with value head h reading key head h // (Hv/Hk)
  (page "GDN CTE Kernel API Reference", Notes).
* :mod:`oracle.chunked` -- an independent chunk-parallel (WY) derivation in
  numpy fp64, used only as a cross-check of :func:`gdn_serial`.
"""
import ctypes
import os

import numpy as np

from . import build as _build

__all__ = ["gdn_serial", "default_threads"]

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
    if state is None:
        st = np.zeros((B, Hv, Dk, Dv), dtype=np.float64)
    elif inplace:
        st = state
        if not (isinstance(st, np.ndarray) and st.dtype == np.float64
                and st.flags.c_contiguous and st.shape == (B, Hv, Dk, Dv)):
            raise ValueError("oracle: inplace needs a C-contiguous float64 state of the right shape")
    else:
        st = np.array(state, dtype=np.float64, order="C", copy=True)
        if st.shape != (B, Hv, Dk, Dv):
            raise ValueError("oracle: bad state shape")
    out = np.empty((B, Hv, S, Dv), dtype=np.float64)
    n = default_threads() if nthreads is None else int(nthreads)
    rc = _lib().oracle_gdn_serial(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, g_log.ctypes.data, beta.ctypes.data,
        float(scale), st.ctypes.data, out.ctypes.data, B, Hk, Hv, S, Dk, Dv, n)
    if rc != 0:
        raise RuntimeError("oracle_gdn_serial failed with code %d" % rc)
    return out, st

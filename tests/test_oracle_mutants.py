"""Sensitivity of the oracle's pins: copies of the oracle's C source with one
planted mistake each (a dropped term, a wrong sign, a wrong index, a
transposed operand, ...) are compiled on the CPU, and every copy must fail at
least one pin. The planted mistakes live only in temporary copies."""
import ctypes
import os
import subprocess
import tempfile
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_serial.c")

MUTANTS = {
    "no_decay": ("St[i * Dv + c] *= a;", "St[i * Dv + c] *= 1.0;"),
    "decay_twice": ("St[i * Dv + c] *= a;", "St[i * Dv + c] *= a * a;"),
    "delta_sign": ("u[c] = be * (vt[c] - x);", "u[c] = be * (vt[c] + x);"),
    "no_beta": ("u[c] = be * (vt[c] - x);", "u[c] = (vt[c] - x);"),
    "no_delta": ("u[c] = be * (vt[c] - x);", "u[c] = be * vt[c];"),
    "gqa_modulo": ("const long j = h / G;", "const long j = h % Hk;"),
    "transposed_read": ("x += St[i * Dv + c] * kt[i];",
                        "x += St[(c % Dk) * Dv + (i % Dv)] * kt[i];"),
    "out_reads_k": ("y += St[i * Dv + c] * qt[i];", "y += St[i * Dv + c] * kt[i];"),
    "no_scale": ("ot[c] = scale * y;", "ot[c] = y;"),
    "write_with_q": ("St[i * Dv + c] += kt[i] * u[c];", "St[i * Dv + c] += qt[i] * u[c];"),
    # the gate and normalisation prologue
    "softplus_sign": (": log1p(exp(x));", ": log1p(exp(-x));"),
    "softplus_no_shift": ("x + log1p(exp(-x))", "log1p(exp(-x))"),
    "gate_no_dt_bias": ("softplus(a + dt_bias_h)", "softplus(a)"),
    "gate_no_exp": ("*g = -exp(A_log_h) *", "*g = -A_log_h *"),
    "gate_sign": ("*g = -exp(A_log_h) *", "*g = exp(A_log_h) *"),
    "sigmoid_sign": ("1.0 / (1.0 + exp(-x));", "1.0 / (1.0 + exp(x));"),
    "norm_no_sqrt": ("1.0 / sqrt(ss + eps);", "1.0 / (ss + eps);"),
    "norm_eps_outside": ("1.0 / sqrt(ss + eps);", "1.0 / (sqrt(ss) + eps);"),
    "q_not_normalised": ("l2norm_row(qt, eps, qd, Dk);",
                         "for (long i = 0; i < Dk; ++i) qd[i] = (double)qt[i];"),
    "k_not_normalised": ("l2norm_row(kt, eps, kd, Dk);",
                         "for (long i = 0; i < Dk; ++i) kd[i] = (double)kt[i];"),
    "gate_key_head": ("(double)A_log[h],", "(double)A_log[j],"),
    "gates_swapped": ("gates((double)gl[bh * S + t], (double)bt[bh * S + t],",
                      "gates((double)bt[bh * S + t], (double)gl[bh * S + t],"),
}


def _build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    path = os.path.join(tmpdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmpdir, name + ".so")
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", path, "-o", lib,
                    "-lm"], check=True)
    return lib


def _wrap(libpath):
    """The mutant's three entries, marshalled like the real oracle's."""
    lib = ctypes.CDLL(libpath)
    real = oracle._lib()
    for name in ("oracle_gdn_serial", "oracle_gdn_serial_gated", "oracle_gdn_gates",
                 "oracle_l2norm"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = getattr(real, name).argtypes
    f32 = lambda *xs: [np.ascontiguousarray(np.asarray(x, np.float32)) for x in xs]

    def state_of(state, B, Hv, Dk, Dv):
        return (np.zeros((B, Hv, Dk, Dv)) if state is None
                else np.array(state, dtype=np.float64, order="C", copy=True))

    def fn(q, k, v, g, beta, scale, state=None):
        q, k, v, g, beta = f32(q, k, v, g, beta)
        B, Hk, S, Dk = q.shape
        Hv, Dv = v.shape[1], v.shape[3]
        st = state_of(state, B, Hv, Dk, Dv)
        out = np.empty((B, Hv, S, Dv))
        rc = lib.oracle_gdn_serial(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                                   beta.ctypes.data, float(scale), st.ctypes.data,
                                   out.ctypes.data, B, Hk, Hv, S, Dk, Dv, 1)
        assert rc == 0
        return out, st

    def gated(q, k, v, a, b, A_log, dt_bias, scale, eps, state=None):
        q, k, v, a, b, A_log, dt_bias = f32(q, k, v, a, b, A_log, dt_bias)
        B, Hk, S, Dk = q.shape
        Hv, Dv = v.shape[1], v.shape[3]
        st = state_of(state, B, Hv, Dk, Dv)
        out = np.empty((B, Hv, S, Dv))
        rc = lib.oracle_gdn_serial_gated(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, a.ctypes.data, b.ctypes.data,
            A_log.ctypes.data, dt_bias.ctypes.data, float(eps), float(scale), st.ctypes.data,
            out.ctypes.data, B, Hk, Hv, S, Dk, Dv, 1)
        assert rc == 0
        return out, st

    def gates(a, b, A_log, dt_bias):
        a, b, A_log, dt_bias = f32(a, b, A_log, dt_bias)
        g = np.empty(a.shape)
        be = np.empty(a.shape)
        assert lib.oracle_gdn_gates(a.ctypes.data, b.ctypes.data, A_log.ctypes.data,
                                    dt_bias.ctypes.data, g.ctypes.data, be.ctypes.data,
                                    *a.shape) == 0
        return g, be

    def l2norm(x, eps):
        (x,) = f32(x)
        y = np.empty(x.shape)
        assert lib.oracle_l2norm(x.ctypes.data, float(eps), y.ctypes.data,
                                 x.size // x.shape[-1], x.shape[-1]) == 0
        return y

    return fn, SimpleNamespace(gated=gated, gates=gates, l2norm=l2norm)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        fn, ns = _wrap(_build_mutant(name, d))
        caught = []
        for pin, arg in [(p, fn) for p in P.ALL_PINS] + [(p, ns) for p in P.GATED_PINS]:
            try:
                pin(arg)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, "planted mistake %r passed every pin" % name


# The conv1d oracle is numpy: its mutants are edited copies of the module
# source, executed as fresh modules.
CONV_SRC = os.path.join(os.path.dirname(oracle.__file__), "conv1d.py")
CONV_MUTANTS = {
    "tap_order": ("lag = K - 1 - j", "lag = j"),
    "lag_off_by_one": ("lag = K - 1 - j", "lag = K - j"),
    "no_silu": ("return silu(y), state", "return y, state"),
    "sigmoid_not_silu": ("return y / (1.0 + np.exp(-y))", "return 1.0 / (1.0 + np.exp(-y))"),
    "state_from_output": ("state[:, :, j] = x[:, :, t]", "state[:, :, j] = y[:, :, t]"),
    "state_off_by_one": ("t = T - K + j\n", "t = T - K + j - 1\n"),
    "decode_shift_wrong": ("window = np.concatenate([state[:, :, 1:], x[:, :, None]], axis=2)",
                           "window = np.concatenate([x[:, :, None], state[:, :, :-1]], axis=2)"),
    "decode_no_silu": ("return silu(y), window", "return y, window"),
    "wrong_channel_weights": ("w[None, :, j, None]", "w[None, ::-1, j, None]"),
    "decode_reversed_taps": ("y += w[None, :, j] * window[:, :, j]",
                             "y += w[None, :, K - 1 - j] * window[:, :, j]"),
}


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(name):
    import types
    old, new = CONV_MUTANTS[name]
    src = open(CONV_SRC).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    mod = types.ModuleType("conv1d_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), mod.__dict__)
    ns = SimpleNamespace(prefill=mod.conv1d_prefill, decode=mod.conv1d_decode)
    caught = []
    for pin in P.CONV_PINS:
        try:
            pin(ns)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name

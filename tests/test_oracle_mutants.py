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
    "f64_inputs_as_float": ("return f64 ? ((const double*)p)[i]", "return 0 ? ((const double*)p)[i]"),
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
    "q_not_normalised": ("l2norm_row(q, qt, f64, eps, qd, Dk);",
                         "for (long i = 0; i < Dk; ++i) qd[i] = in_at(q, qt + i, f64);"),
    "k_not_normalised": ("l2norm_row(k, kt, f64, eps, kd, Dk);",
                         "for (long i = 0; i < Dk; ++i) kd[i] = in_at(k, kt + i, f64);"),
    "gate_key_head": ("in_at(A_log, h, f64)", "in_at(A_log, j, f64)"),
    "gates_swapped": ("gates(in_at(gl, bh * S + t, f64), in_at(bt, bh * S + t, f64),",
                      "gates(in_at(bt, bh * S + t, f64), in_at(gl, bh * S + t, f64),"),
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
    for name in ("oracle_gdn_serial", "oracle_gdn_serial_gated", "oracle_gdn_serial_gated_f64",
                 "oracle_gdn_gates", "oracle_l2norm"):
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

    def gated_f64(q, k, v, a, b, A_log, dt_bias, scale, eps, state=None):
        q, k, v, a, b, A_log, dt_bias = [np.ascontiguousarray(np.asarray(x, np.float64))
                                         for x in (q, k, v, a, b, A_log, dt_bias)]
        B, Hk, S, Dk = q.shape
        Hv, Dv = v.shape[1], v.shape[3]
        st = state_of(state, B, Hv, Dk, Dv)
        out = np.empty((B, Hv, S, Dv))
        rc = lib.oracle_gdn_serial_gated_f64(
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

    return fn, SimpleNamespace(gated=gated, gated_f64=gated_f64, gates=gates, l2norm=l2norm)


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


BLOCK_SRC = os.path.join(os.path.dirname(oracle.__file__), "block.py")
BLOCK_MUTANTS = {
    "rms_no_sqrt": ("return o / np.sqrt(ms + eps)", "return o / (ms + eps)"),
    "rms_sum_not_mean": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                         "ms = np.sum(o * o, axis=-1, keepdims=True)"),
    "gate_sigmoid_not_silu": ("* (z / (1.0 + np.exp(-z)))", "* (1.0 / (1.0 + np.exp(-z)))"),
    "no_weight": ("/ np.sqrt(ms + eps) * weight *", "/ np.sqrt(ms + eps) *"),
    "q_k_swapped": ("q = xc[:, :Hk * Dk].reshape(B, Hk, 1, Dk)",
                    "q = xc[:, Hk * Dk:2 * Hk * Dk].reshape(B, Hk, 1, Dk)"),
    "v_from_k": ("v = xc[:, 2 * Hk * Dk:].reshape(B, Hv, 1, Dv)",
                 "v = xc[:, Hk * Dk:Hk * Dk + Hv * Dv].reshape(B, Hv, 1, Dv)"),
    "z_not_applied": ("np.asarray(z, np.float64).reshape(B, Hv, Dv)",
                      "np.ones((B, Hv, Dv)) * 30.0"),
}


@pytest.mark.parametrize("name", sorted(BLOCK_MUTANTS))
def test_block_mutant_is_caught(name):
    import types
    old, new = BLOCK_MUTANTS[name]
    src = open(BLOCK_SRC).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    mod = types.ModuleType("block_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), mod.__dict__)
    ns = SimpleNamespace(rmsnorm=mod.rmsnorm_gated, block=mod.decode_block)
    caught = []
    for pin in P.RMS_PINS:
        try:
            pin(ns)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name

"""Sensitivity of the oracle's pins: copies of the oracle's C source with one
planted mistake each (a dropped term, a wrong sign, a wrong index, a
transposed operand, ...) are compiled on the CPU, and every copy must fail at
least one pin. The planted mistakes live only in temporary copies."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_serial.c")

MUTANTS = {
    "no_decay": ("St[i * Dv + c] *= a;", "St[i * Dv + c] *= 1.0;"),
    "decay_twice": ("St[i * Dv + c] *= a;", "St[i * Dv + c] *= a * a;"),
    "delta_sign": ("u[c] = be * ((double)vt[c] - x);", "u[c] = be * ((double)vt[c] + x);"),
    "no_beta": ("u[c] = be * ((double)vt[c] - x);", "u[c] = ((double)vt[c] - x);"),
    "no_delta": ("u[c] = be * ((double)vt[c] - x);", "u[c] = be * (double)vt[c];"),
    "gqa_modulo": ("const long j = h / G;", "const long j = h % Hk;"),
    "transposed_read": ("x += St[i * Dv + c] * (double)kt[i];",
                        "x += St[(c % Dk) * Dv + (i % Dv)] * (double)kt[i];"),
    "out_reads_k": ("y += St[i * Dv + c] * (double)qt[i];", "y += St[i * Dv + c] * (double)kt[i];"),
    "no_scale": ("ot[c] = scale * y;", "ot[c] = y;"),
    "write_with_q": ("St[i * Dv + c] += (double)kt[i] * u[c];",
                     "St[i * Dv + c] += (double)qt[i] * u[c];"),
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
    lib = ctypes.CDLL(libpath)
    f = lib.oracle_gdn_serial
    f.restype = ctypes.c_int
    f.argtypes = oracle._lib().oracle_gdn_serial.argtypes

    def fn(q, k, v, g, beta, scale, state=None):
        q, k, v, g, beta = (np.ascontiguousarray(np.asarray(a, np.float32))
                            for a in (q, k, v, g, beta))
        B, Hk, S, Dk = q.shape
        Hv, Dv = v.shape[1], v.shape[3]
        st = (np.zeros((B, Hv, Dk, Dv)) if state is None
              else np.array(state, dtype=np.float64, order="C", copy=True))
        out = np.empty((B, Hv, S, Dv))
        rc = f(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data, beta.ctypes.data,
               float(scale), st.ctypes.data, out.ctypes.data, B, Hk, Hv, S, Dk, Dv, 1)
        assert rc == 0
        return out, st
    return fn


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        fn = _wrap(_build_mutant(name, d))
        caught = []
        for pin in P.ALL_PINS:
            try:
                pin(fn)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, "planted mistake %r passed every pin" % name

"""The CPU oracle against facts the mathematics fixes (closed forms, hand-worked
examples, brute-force products, the chunked derivation, invariants)."""
import numpy as np
import pytest

import oracle
from oracle.chunked import chunk_terms
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.gdn_serial)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_chunked_form(pin):
    """The chunked derivation satisfies the same pins (it is the cross-check)."""
    from oracle.chunked import gdn_chunked
    pin(lambda *a: gdn_chunked(*a, chunk=4))


def test_thread_count_does_not_change_result():
    q, k, v, g, beta, s0 = P.random_case(20, B=3, Hk=2, Hv=4, S=33, Dk=8, Dv=8)
    o1, s1 = oracle.gdn_serial(q, k, v, g, beta, 0.5, s0, nthreads=1)
    o2, s2 = oracle.gdn_serial(q, k, v, g, beta, 0.5, s0, nthreads=7)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_inverse_is_exact():
    """T = (I + A)^{-1} of the chunked form: (I + A) T = I and T is unit lower
    triangular; with normalised keys max|T| stays O(1)."""
    q, k, v, g, beta, _ = P.random_case(21, S=64, Dk=16, Dv=8, decay=0.01)
    t = chunk_terms(k[0, 0].astype(np.float64), v[0, 0].astype(np.float64),
                    g[0, 0].astype(np.float64), beta[0, 0].astype(np.float64))
    T, A = t["T"], t["A"]
    assert np.allclose((np.eye(64) + A) @ T, np.eye(64), atol=1e-12)
    assert np.allclose(np.triu(T, 1), 0.0) and np.allclose(np.diag(T), 1.0)
    assert np.max(np.abs(T)) < 4.0


def test_zero_length_and_strong_decay():
    q, k, v, g, beta, s0 = P.random_case(22, S=0)
    o, s = oracle.gdn_serial(q, k, v, g, beta, 1.0, s0)
    assert o.shape == (1, 1, 0, 3) and np.array_equal(s, s0.astype(np.float64))
    # decay so strong that e^{gamma} underflows in a 64-token chunk: no inf/nan
    q, k, v, g, beta, s0 = P.random_case(23, S=64, decay=40.0)
    o, s = oracle.gdn_serial(q, k, v, g, beta, 1.0, s0)
    from oracle.chunked import gdn_chunked
    oc, sc = gdn_chunked(q, k, v, g, beta, 1.0, s0, chunk=64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(oc))
    assert np.allclose(o, oc, atol=1e-12) and np.allclose(s, sc, atol=1e-12)


def test_workload_inputs_are_seeded_and_normalised():
    import workloads
    w = workloads.WORKLOADS["tiny_f32"]
    a = workloads.draw_workload(w)
    b = workloads.draw_workload(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
    n = np.linalg.norm(a["q"].astype(np.float64), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-6)
    assert np.all(a["g_log"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))
    # bf16 rounding: round-to-nearest-even on the upper 16 bits
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.00390625], np.float32)
    r = workloads.bf16_round(x)
    assert list(r) == [1.0, 1.0 + 4 * 2.0 ** -8, -2.5, 1.0]


@pytest.mark.parametrize("pin", P.GATED_PINS, ids=lambda f: f.__name__)
def test_gated_pin(pin):
    from types import SimpleNamespace
    pin(SimpleNamespace(gated=oracle.gdn_serial_gated, gated_f64=oracle.gdn_serial_gated_f64,
                        gates=oracle.gdn_gates, l2norm=oracle.l2_normalize))


@pytest.mark.parametrize("pin", P.CONV_PINS, ids=lambda f: f.__name__)
def test_conv_pin(pin):
    from types import SimpleNamespace
    from oracle import conv1d
    pin(SimpleNamespace(prefill=conv1d.conv1d_prefill, decode=conv1d.conv1d_decode))


@pytest.mark.parametrize("pin", P.RMS_PINS, ids=lambda f: f.__name__)
def test_rms_block_pin(pin):
    from types import SimpleNamespace
    from oracle import block
    pin(SimpleNamespace(rmsnorm=block.rmsnorm_gated, block=block.decode_block))

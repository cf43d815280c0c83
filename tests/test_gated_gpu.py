"""The gated entry points (gate and L2-norm prologue on the device) against
the fp64 oracle's gated recurrence, element by element: the named workloads
with raw inputs, edge shapes, an epsilon that matters, all-zero key rows,
strong decay, and decode steps chained over a carried state."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check, log, to_np, upload_raw

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
EPS = 1e-6


def _run(d, dtype, scale, eps):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    t = upload_raw(d, dtype)
    out = gdn.chunked_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                    t["dt_bias"], scale, eps, t["state"])
    torch.cuda.synchronize()
    return to_np(out), to_np(t["state"])


def _parity(name, d, dtype, scale, eps=EPS):
    log("gated prefill parity:", name, "eps", eps,
        {k: v.shape for k, v in d.items() if v is not None and k in ("q_raw", "v")})
    out, st = _run(d, dtype, scale, eps)
    ro, rs = oracle.gdn_serial_gated(d["q_raw"], d["k_raw"], d["v"], d["a"], d["b"],
                                     d["A_log"], d["dt_bias"], scale, eps, d["state"])
    return check(name, dtype, out, ro, st, rs)


def test_gated_tiny_f32():
    w = W["tiny_f32"]
    _parity(w.name, workloads.draw_workload(w, raw=True), "f32", w.scale)


def test_gated_prefill_s2048():
    w = W["prefill_s2048"]
    _parity(w.name, workloads.draw_workload(w, raw=True), "bf16", w.scale)


def test_gated_prefill_b4_s8192_full():
    """The bench workload with raw inputs, in the configuration the bench times."""
    w = W["prefill_b4_s8192"]
    _parity(w.name, workloads.draw_workload(w, raw=True), "bf16", w.scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_strong_decay(dtype):
    w = W["prefill_s65536"]
    d = workloads.draw_prefill(B=1, Hk=4, Hv=8, S=4096, Dk=128, Dv=128, dtype=dtype,
                            state="normal", decay="strong", seed=(4, 1, 16), raw=True)
    _parity("strong/%s" % dtype, d, dtype, w.scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [
    dict(B=1, Hk=2, Hv=2, S=64, Dk=64, Dv=64),      # one chunk, G = 1
    dict(B=2, Hk=1, Hv=4, S=192, Dk=128, Dv=128),   # G = 4
    dict(B=1, Hk=2, Hv=4, S=256, Dk=80, Dv=48),     # padded Dk, ragged value slice
    dict(B=3, Hk=3, Hv=3, S=128, Dk=16, Dv=112),    # smallest Dk
    dict(B=1, Hk=1, Hv=2, S=320, Dk=128, Dv=16),    # smallest Dv
])
def test_gated_shapes(dtype, shape):
    d = workloads.draw_prefill(dtype=dtype, state="normal", decay="weak", seed=(9, 2, 11),
                            raw=True, **shape)
    _parity("gated shape %s %s" % (dtype, shape), d, dtype, 1.0 / np.sqrt(shape["Dk"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_epsilon_matters(dtype):
    """Short raw q, k (|x|^2 ~ 0.3) with eps = 0.1: the epsilon changes every
    normalised vector by several percent, so its placement is tested."""
    d = workloads.draw_prefill(B=1, Hk=2, Hv=4, S=256, Dk=128, Dv=64, dtype=dtype,
                            state="normal", seed=(9, 0, 12), raw=True)
    for key in ("q_raw", "k_raw"):
        d[key] = (d[key] * np.float32(0.05))
        if dtype == "bf16":
            d[key] = workloads.bf16_round(d[key])
    _parity("eps=0.1 %s" % dtype, d, dtype, 0.125, eps=0.1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_zero_key_rows(dtype):
    """All-zero raw keys (and queries) normalise to zero with eps > 0: those
    tokens only decay the state."""
    d = workloads.draw_prefill(B=1, Hk=1, Hv=2, S=128, Dk=128, Dv=128, dtype=dtype,
                            state="normal", seed=(9, 0, 13), raw=True)
    d["k_raw"][:, :, 5:40:7] = 0.0
    d["q_raw"][:, :, 64:70] = 0.0
    _parity("zero rows %s" % dtype, d, dtype, 0.1)


def _decode_steps(w, nsteps, dtype, eps=EPS, **over):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    state0, steps = workloads.draw_decode_steps(w, nsteps=nsteps, raw=True, **over)
    st_dev = torch.from_numpy(state0).cuda()
    st_ref = state0.astype(np.float64)
    outs, refs = [], []
    for d in steps:
        t = upload_raw(d, dtype)
        o = gdn.decode_step_gated(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                                  t["a"][:, :, 0].contiguous(), t["b"][:, :, 0].contiguous(),
                                  t["A_log"], t["dt_bias"], w.scale, eps, st_dev)
        outs.append(to_np(o))
        ro, st_ref = oracle.gdn_serial_gated(d["q_raw"], d["k_raw"], d["v"], d["a"], d["b"],
                                             d["A_log"], d["dt_bias"], w.scale, eps, st_ref,
                                             inplace=True)
        refs.append(ro[:, :, 0])
    torch.cuda.synchronize()
    return np.stack(outs), np.stack(refs), to_np(st_dev), st_ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [dict(B=3, Hk=2, Hv=4, Dk=128, Dv=128),
                                   dict(B=2, Hk=1, Hv=3, Dk=64, Dv=32),
                                   dict(B=2, Hk=2, Hv=2, Dk=48, Dv=80)])
def test_gated_decode_small(dtype, shape):
    w = W["decode_b256"]
    log("gated decode small", dtype, shape)
    o, ro, s, rs = _decode_steps(w, 8, dtype, **shape)
    check("gated decode %s %s" % (dtype, shape), dtype, o, ro, s, rs)


def test_gated_decode_b256_64_steps():
    w = W["decode_b256"]
    log("gated decode_b256 x 64 steps")
    o, ro, s, rs = _decode_steps(w, w.steps, "bf16")
    check("gated decode_b256 64 steps", "bf16", o, ro, s, rs)


def test_gated_decode_epsilon_matters():
    w = W["decode_b256"]
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    state0, steps = workloads.draw_decode_steps(w, nsteps=4, raw=True, B=2, Hk=2, Hv=4)
    st_dev = torch.from_numpy(state0).cuda()
    st_ref = state0.astype(np.float64)
    outs, refs = [], []
    for d in steps:
        for key in ("q_raw", "k_raw"):
            d[key] = workloads.bf16_round(d[key] * np.float32(0.05))
        t = upload_raw(d, "bf16")
        outs.append(to_np(gdn.decode_step_gated(
            t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0], t["a"][:, :, 0].contiguous(),
            t["b"][:, :, 0].contiguous(), t["A_log"], t["dt_bias"], w.scale, 0.1, st_dev)))
        ro, st_ref = oracle.gdn_serial_gated(d["q_raw"], d["k_raw"], d["v"], d["a"], d["b"],
                                             d["A_log"], d["dt_bias"], w.scale, 0.1, st_ref,
                                             inplace=True)
        refs.append(ro[:, :, 0])
    torch.cuda.synchronize()
    check("gated decode eps=0.1", "bf16", np.stack(outs), np.stack(refs), to_np(st_dev), st_ref)


def test_gated_decode_iterated_matches_gated_prefill():
    """64 gated decode steps from a state and one 64-token gated prefill from
    it both match the oracle."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=2, Hk=2, Hv=4, S=64, Dk=128, Dv=128, dtype="bf16",
                            state="normal", decay="weak", seed=(9, 2, 14), raw=True)
    t = upload_raw(d, "bf16")
    st_p = t["state"].clone()
    o_p = gdn.chunked_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                    t["dt_bias"], 0.1, EPS, st_p)
    st_d = t["state"].clone()
    outs = []
    for i in range(64):
        c = lambda x: x[:, :, i].contiguous()
        outs.append(gdn.decode_step_gated(c(t["q"]), c(t["k"]), c(t["v"]), c(t["a"]), c(t["b"]),
                                          t["A_log"], t["dt_bias"], 0.1, EPS, st_d))
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_serial_gated(d["q_raw"], d["k_raw"], d["v"], d["a"], d["b"], d["A_log"],
                                     d["dt_bias"], 0.1, EPS, d["state"])
    check("gated prefill vs oracle", "bf16", to_np(o_p), ro, to_np(st_p), rs)
    check("gated decode x64 vs oracle", "bf16", to_np(torch.stack(outs, dim=2)), ro,
          to_np(st_d), rs)


def test_gated_error_writes_nothing():
    """A negative epsilon is refused before anything is launched."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=1, Hk=1, Hv=1, S=64, Dk=64, Dv=64, dtype="bf16",
                            state="normal", seed=(9, 0, 15), raw=True)
    t = upload_raw(d, "bf16")
    out = torch.full((1, 1, 64, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    st = t["state"].clone()
    with pytest.raises(gdn.GdnError) as e:
        gdn.chunked_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                  t["dt_bias"], 0.1, -1.0, st, out=out)
    assert e.value.code == 9
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.equal(st, t["state"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_gated_ragged_sequence_length(dtype, eps):
    """A partial last chunk with the prologue on the device: the missing
    tokens' gates are zero and their (zero) rows get no norm factor, also
    with eps = 0."""
    d = workloads.draw_prefill(B=1, Hk=2, Hv=4, S=71, Dk=128, Dv=64, dtype=dtype, state="normal",
                            seed=(9, 4, 71), raw=True)
    _parity("gated ragged S=71 %s eps=%g" % (dtype, eps), d, dtype, 0.125, eps=eps)

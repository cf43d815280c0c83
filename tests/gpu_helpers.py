"""Helpers for the GPU parity tests: upload seeded inputs, run the library,
and measure the error against the oracle.

Error metric (one number per tensor, the oracle tensor's RMS over the whole
tensor as the yardstick):

    E(x) = max_i |x_i - ref_i| / rms(ref)

Limits: fp32 operands 1e-4 for out and state; bf16 operands 2e-2 for out and
1e-2 for state. The state is always fp32 and is held to E itself.

A bf16 output is first rounded to bf16 (round to nearest even), the output
format the prefill interface prescribes; that rounding alone moves an element
by up to half a bf16 ulp, at most 2^-8 |x|. Outputs reach ~20x their RMS on
these workloads, so the rounded exact result would already score ~5e-2 in E.
For bf16 outputs the element-wise allowance of that half ulp is taken off
first:

    E_bf16(x) = max_i max(0, |x_i - ref_i| - 2^-8 |ref_i|) / rms(ref)

The earlier hybrid form max_i |x_i - ref_i| / (rms(ref) + |ref_i|) is logged
as a secondary figure, not asserted.
"""
import sys

import numpy as np

TOL = {"f32": {"out": 1e-4, "state": 1e-4}, "bf16": {"out": 2e-2, "state": 1e-2}}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


BF16_HALF_ULP = 2.0 ** -8      # bound of |bf16(x) - x| / |x| under round to nearest even


def _rms(ref):
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def rms_err(x, ref):
    """max_i |x_i - ref_i| / rms(ref): the asserted metric for the state and
    for fp32 outputs."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    rms = _rms(ref)
    d = float(np.max(np.abs(x - ref)))
    if rms == 0.0:
        return d
    return d / rms


def bf16_out_err(x, ref):
    """max_i max(0, |x_i - ref_i| - 2^-8 |ref_i|) / rms(ref): the asserted
    metric for outputs stored in bf16 (one half ulp of the output format
    allowed per element)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    excess = np.maximum(np.abs(x - ref) - BF16_HALF_ULP * np.abs(ref), 0.0)
    rms = _rms(ref)
    return float(np.max(excess)) / rms if rms > 0.0 else float(np.max(excess))


def out_err(x, ref, dtype):
    """The asserted output metric of a tensor stored in ``dtype``."""
    return bf16_out_err(x, ref) if dtype == "bf16" else rms_err(x, ref)


def hybrid_err(x, ref):
    """max_i |x_i - ref_i| / (rms(ref) + |ref_i|) (logged, not asserted)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    den = _rms(ref) + np.abs(ref)
    num = np.abs(x - ref)
    ok = den > 0
    return float(np.max(num[ok] / den[ok])) if np.any(ok) else float(np.max(num))


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def upload(d, dtype, device="cuda"):
    """numpy float32 inputs -> device tensors (q, k, v in the compute dtype)."""
    import torch
    td = torch_dtype(dtype)
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(device=device, dtype=td)
    for key in ("g_log", "beta"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(device)
    st = d.get("state")
    if st is not None:
        out["state"] = torch.from_numpy(np.ascontiguousarray(st)).to(device)
    return out


def to_np(t):
    return t.detach().float().cpu().numpy()


def run_prefill(d, dtype, scale, inverse=None):
    """Run gdn_chunked_prefill (or gdn_chunked_prefill_inverse) on the inputs
    of ``d``; returns (out, state) numpy."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    t = upload(d, dtype)
    out = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], scale, t["state"],
                              inverse=inverse)
    torch.cuda.synchronize()
    return to_np(out), to_np(t["state"])


def check(name, dtype, out, ref_out, st, ref_st, tol=None):
    """Asserts out_err(out) and rms_err(state) within the limits of ``dtype``."""
    tol = tol or TOL[dtype]
    eo, es = out_err(out, ref_out, dtype), rms_err(st, ref_st)
    log("  %-40s out err %.3e (tol %.0e)  state err %.3e (tol %.0e)"
        "  [max/rms out %.3e; hybrid out %.3e state %.3e]"
        % (name, eo, tol["out"], es, tol["state"], rms_err(out, ref_out),
           hybrid_err(out, ref_out), hybrid_err(st, ref_st)))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(st)), name + ": non-finite values"
    assert eo <= tol["out"], "%s: out error %.3e > %.0e" % (name, eo, tol["out"])
    assert es <= tol["state"], "%s: state error %.3e > %.0e" % (name, es, tol["state"])
    return eo, es


def upload_raw(d, dtype, device="cuda"):
    """Raw prologue inputs of a draw with ``raw=True`` -> device tensors:
    q, k (un-normalised) and v in the compute dtype; a, b, A_log, dt_bias and
    the state in fp32."""
    import torch
    td = torch_dtype(dtype)
    out = {}
    for key, src in (("q", "q_raw"), ("k", "k_raw"), ("v", "v")):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[src])).to(device=device, dtype=td)
    for key in ("a", "b", "A_log", "dt_bias"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(device)
    if d.get("state") is not None:
        out["state"] = torch.from_numpy(np.ascontiguousarray(d["state"])).to(device)
    return out

"""Seeded synthetic inputs for the gated delta-rule path.

This module only draws inputs; it holds none of the recurrence's arithmetic.
Both the GPU path (through the tests and the bench) and the CPU oracle are fed
from the same arrays drawn here.

Recipe (per workload; ``rng(x) = numpy.random.default_rng(x)``):

1. once per workload and variant, from ``rng([workload_id, variant])``:
   ``A_log[Hv]`` ~ U(log lo, log hi) with (lo, hi) = (1, 16) standard,
   (8, 64) strong decay, (0.01, 0.1) weak decay; ``dt_bias[Hv]`` ~ U(-1, 1).

Then per call, from ``rng([workload_id, variant, step])``, in this order:

2. q, k ``[B,Hk,S,Dk]`` ~ N(0, 1) in float32, L2-normalised per token and head
   (the pages require normalised q/k: "GDN CTE Kernel API Reference", Notes).
3. v ``[B,Hv,S,Dv]`` ~ N(0, 1).
4. a, b ``[B,Hv,S]`` ~ N(0, 1); the gates that a decode block derives from its
   projections ("GDN Block TKG Kernel API Reference", Parameters A_log and
   dt_bias) are g_log = -exp(A_log[h]) softplus(a + dt_bias[h]) and
   beta = sigmoid(b), evaluated in float64 and stored float32.
5. the initial state ``[B,Hv,Dk,Dv]`` ~ N(0, 0.02^2) where the workload carries
   one, else zeros.

For bf16 workloads q, k and v are rounded to bf16 (round to nearest even)
after normalisation; the arrays returned here are float32 holding exactly those
bf16 values, so the oracle sees precisely what the GPU sees.

With ``raw=True`` the draw also returns the quantities before step 2's
normalisation and step 4's gate functions, for the entry points that take the
prologue on the device: ``q_raw``, ``k_raw`` (the N(0, 1) draws of step 2,
rounded to bf16 for bf16 workloads), ``a``, ``b`` (step 4, float32) and
``A_log``, ``dt_bias`` (step 1, float32). They come from the same random
stream, so raw and derived inputs describe the same tokens.

Depthwise conv1d inputs (:func:`draw_conv`), from ``rng([100, B, C, T, K,
step])``: the raw mixed tensor ``[B, C, T]`` ~ N(0, 1) (rounded to bf16 for
bf16), weights ``[C, K]`` ~ U(-1/sqrt(K), 1/sqrt(K)) in float32 (the default
initialisation of a depthwise convolution with K taps), and for decode a
window state ``[B, C, K]`` ~ N(0, 1) and one token ``[B, C]`` per step. The
mixed tensor of the prefill workloads has C = 2 Hk Dk + Hv Dv channels (q|k|v,
"GDN Block TKG Kernel API Reference", Dimensions) and T = S tokens.

Decode-block inputs (:func:`draw_block`), from ``rng([200, B, Hk, Hv, Dk, Dv,
K, step])``: the raw mixed token ``[B, C]`` and the gate ``z [B, Hv Dv]`` ~
N(0, 1), ``a, b [B, Hv]`` ~ N(0, 1) (float32), the conv window ``[B, C, K]``
~ N(0, 1), conv weights as above, ``norm_weight [Dv]`` ~ 1 + N(0, 0.1^2), the
recurrent state ~ N(0, 0.02^2); ``A_log``, ``dt_bias`` as in step 1 (standard
decay) from ``rng([200, Hv])``. Operand tensors (mixed, z, window) are
bf16-exact for bf16.
"""
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "bf16_round", "draw_prefill", "draw_workload",
           "draw_decode_steps", "ConvWorkload", "CONV_WORKLOADS", "draw_conv", "draw_block"]

_DECAY = {"std": (1.0, 16.0), "strong": (8.0, 64.0), "weak": (0.01, 0.1)}
_VARIANT_ID = {"std": 0, "strong": 1, "weak": 2}


@dataclass(frozen=True)
class Workload:
    """A named workload: shapes, operand dtype, initial-state kind."""
    wid: int
    name: str
    B: int
    Hk: int
    Hv: int
    S: int
    Dk: int
    Dv: int
    dtype: str               # "bf16" or "f32" (q, k, v, out)
    state: str               # "zero" or "normal"
    steps: int = 0           # >0: decode workload, S == 1 per step
    variants: tuple = field(default=("std",))

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.Dk))


WORKLOADS = {
    w.name: w for w in (
        Workload(0, "tiny_f32", 1, 2, 2, 128, 64, 64, "f32", "zero"),
        Workload(1, "prefill_s2048", 1, 16, 32, 2048, 128, 128, "bf16", "zero"),
        Workload(2, "prefill_b4_s8192", 4, 16, 32, 8192, 128, 128, "bf16", "normal"),
        Workload(3, "decode_b256", 256, 16, 32, 1, 128, 128, "bf16", "normal", steps=64),
        Workload(4, "prefill_s65536", 1, 16, 32, 65536, 128, 128, "bf16", "normal",
                 variants=("std", "strong")),
    )
}


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def _l2norm(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _head_params(decay, Hv, seed):
    rng = np.random.default_rng(list(seed))
    lo, hi = _DECAY[decay]
    A_log = rng.uniform(np.log(lo), np.log(hi), size=Hv)
    dt_bias = rng.uniform(-1.0, 1.0, size=Hv)
    return A_log, dt_bias


def draw_prefill(B, Hk, Hv, S, Dk, Dv, dtype="bf16", state="zero", decay="std",
                 seed=(0, 0, 0), raw=False):
    """Draw one prefill batch. Returns a dict of float32 numpy arrays:
    q, k [B,Hk,S,Dk]; v [B,Hv,S,Dv]; g_log, beta [B,Hv,S]; state [B,Hv,Dk,Dv]
    (zeros for ``state="zero"``, None for ``state="none"``); with ``raw`` also
    q_raw, k_raw, a, b, A_log, dt_bias (see the module docstring).
    ``seed`` is (workload_id, variant, step); the per-head gate parameters
    come from (workload_id, variant) alone."""
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    A_log, dt_bias = _head_params(decay, Hv, seed[:2])
    rng = np.random.default_rng(list(seed))
    q_raw = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    k_raw = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    q, k = _l2norm(q_raw), _l2norm(k_raw)
    v = rng.standard_normal((B, Hv, S, Dv), dtype=np.float32)
    a = rng.standard_normal((B, Hv, S))
    b = rng.standard_normal((B, Hv, S))
    x = a + dt_bias[None, :, None]
    softplus = np.logaddexp(0.0, x)
    g_log = (-np.exp(A_log)[None, :, None] * softplus).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    if state == "normal":
        st = (0.02 * rng.standard_normal((B, Hv, Dk, Dv))).astype(np.float32)
    elif state == "zero":
        st = np.zeros((B, Hv, Dk, Dv), dtype=np.float32)
    elif state == "none":
        st = None
    else:
        raise ValueError("state must be 'zero', 'normal' or 'none'")
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    d = {"q": q, "k": k, "v": v, "g_log": g_log, "beta": beta, "state": st}
    if raw:
        if dtype == "bf16":
            q_raw, k_raw = bf16_round(q_raw), bf16_round(k_raw)
        d.update(q_raw=q_raw, k_raw=k_raw, a=a.astype(np.float32), b=b.astype(np.float32),
                 A_log=A_log.astype(np.float32), dt_bias=dt_bias.astype(np.float32))
    return d


def draw_workload(w, variant="std", step=0, state=None, **overrides):
    """Draw the inputs of a named :class:`Workload` (optionally with shape
    overrides such as ``B=2`` for reduced parity runs)."""
    shp = dict(B=w.B, Hk=w.Hk, Hv=w.Hv, S=w.S, Dk=w.Dk, Dv=w.Dv)
    shp.update(overrides)
    return draw_prefill(dtype=w.dtype, state=w.state if state is None else state,
                        decay=variant, seed=(w.wid, _VARIANT_ID[variant], step), **shp)


def draw_decode_steps(w, nsteps=None, variant="std", **overrides):
    """Draw a decode workload: the initial state (from step 0's draw) and, for
    each of ``nsteps`` steps i, one token of q, k, v, g_log, beta drawn with
    step = i + 1. Returns (state [B,Hv,Dk,Dv], list of per-step dicts, S == 1)."""
    n = w.steps if nsteps is None else nsteps
    state = draw_workload(w, variant=variant, step=0, S=1, **overrides)["state"]
    steps = []
    for i in range(n):
        d = draw_workload(w, variant=variant, step=i + 1, S=1, state="none", **overrides)
        del d["state"]
        steps.append(d)
    return state, steps


@dataclass(frozen=True)
class ConvWorkload:
    """A depthwise conv1d workload: batch, channels, tokens (1 = decode), taps."""
    name: str
    B: int
    C: int
    T: int
    K: int
    dtype: str


CONV_WORKLOADS = {
    w.name: w for w in (
        # the mixed q|k|v tensor of the B=4, S=8192 prefill (C = 2*16*128 + 32*128)
        ConvWorkload("conv_prefill_b4_t8192", 4, 8192, 8192, 4, "bf16"),
        # one decode token for the B=256 decode batch
        ConvWorkload("conv_decode_b256", 256, 8192, 1, 4, "bf16"),
    )
}


def draw_conv(B, C, T, K, dtype="bf16", step=0, decode=False):
    """Draw conv1d inputs. Returns float32 arrays: ``x`` [B, C, T] (decode:
    [B, C]), ``w`` [C, K], and for decode ``state`` [B, C, K]; bf16-exact
    for dtype bf16."""
    rng = np.random.default_rng([100, B, C, T, K, step])
    w = rng.uniform(-1.0, 1.0, (C, K)).astype(np.float32) / np.float32(np.sqrt(K))
    if decode:
        x = rng.standard_normal((B, C), dtype=np.float32)
        st = rng.standard_normal((B, C, K), dtype=np.float32)
        if dtype == "bf16":
            x, st = bf16_round(x), bf16_round(st)
        return {"x": x, "w": w, "state": st}
    x = rng.standard_normal((B, C, T), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    return {"x": x, "w": w}


def draw_block(B, Hk, Hv, Dk, Dv, K=4, dtype="bf16", step=0, with_state=True):
    """Inputs of one decode-block token (see the module docstring). Returns a
    dict of float32 arrays: mixed, z, a, b, conv_state, conv_weight, A_log,
    dt_bias, norm_weight, state (step > 0 with ``with_state=False`` omits the
    window, the weights and the states, which carry over between steps)."""
    C = 2 * Hk * Dk + Hv * Dv
    rng = np.random.default_rng([200, B, Hk, Hv, Dk, Dv, K, step])
    d = {"mixed": rng.standard_normal((B, C), dtype=np.float32),
         "z": rng.standard_normal((B, Hv * Dv), dtype=np.float32),
         "a": rng.standard_normal((B, Hv), dtype=np.float32),
         "b": rng.standard_normal((B, Hv), dtype=np.float32)}
    if with_state:
        d["conv_state"] = rng.standard_normal((B, C, K), dtype=np.float32)
        d["conv_weight"] = (rng.uniform(-1.0, 1.0, (C, K)) / np.sqrt(K)).astype(np.float32)
        d["norm_weight"] = (1.0 + 0.1 * rng.standard_normal(Dv)).astype(np.float32)
        d["state"] = (0.02 * rng.standard_normal((B, Hv, Dk, Dv))).astype(np.float32)
        A_log, dt_bias = _head_params("std", Hv, (200, Hv))
        d["A_log"], d["dt_bias"] = A_log.astype(np.float32), dt_bias.astype(np.float32)
    if dtype == "bf16":
        for key in ("mixed", "z", "conv_state"):
            if key in d:
                d[key] = bf16_round(d[key])
    return d

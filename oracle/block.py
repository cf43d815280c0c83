"""RMSNormGated and the decode block without its projections -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library shares no code with it.

* :func:`rmsnorm_gated` -- the output epilogue the "GDN Block TKG Kernel API
  Reference" page names (introduction: "RMSNormGated"; Parameters
  norm_weight, the gamma of RMSNormGated over head_v_dim; W_in_z, whose
  projection z gates it). The page gives no formula or epsilon. Read as the
  gated RMS norm over each head's Dv outputs, normalise first:
      y = o / sqrt(mean_d(o_d^2) + eps) * gamma_d * silu(z_d),
  silu(z) = z / (1 + e^{-z}), with eps an argument.
* :func:`decode_block` -- the page's decode layer between its input and output
  projections (introduction): the conv1d decode step over the raw mixed
  q|k|v token ("GDN Conv1D Kernel API Reference"), the split into q, k (Hk
  heads of Dk) and v (Hv heads of Dv) in that channel order (Dimensions:
  conv_dim = 2 key_dim + value_dim), the gate and normalisation prologue, the
  single-token recurrence and RMSNormGated. Composed from the other oracle
  functions, each pinned on its own.

float64 throughout.
"""
import numpy as np

import oracle
from oracle import conv1d

__all__ = ["rmsnorm_gated", "decode_block"]


def rmsnorm_gated(o, z, weight, eps):
    """o, z [..., D]; weight [D]. Returns o / sqrt(mean(o^2) + eps) * weight *
    silu(z) over the last axis, float64."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    if o.shape != z.shape or weight.shape != (o.shape[-1],):
        raise ValueError("oracle: rmsnorm_gated shapes")
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * weight * (z / (1.0 + np.exp(-z)))


def decode_block(mixed, z, a, b, conv_state, conv_weight, A_log, dt_bias, norm_weight,
                 state, scale, l2_eps, norm_eps, Hk, Hv, Dk, Dv, inplace=False):
    """One decode token through the block without projections.

    mixed [B, C] raw q|k|v token (C = 2 Hk Dk + Hv Dv); z [B, Hv Dv]; a, b
    [B, Hv]; conv_state [B, C, K]; conv_weight [C, K]; A_log, dt_bias [Hv];
    norm_weight [Dv]; state [B, Hv, Dk, Dv]. Returns (out [B, Hv Dv],
    new conv_state [B, C, K], new state), float64.
    """
    mixed = np.asarray(mixed, dtype=np.float32)
    B, C = mixed.shape
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError("oracle: mixed must hold q|k|v channels")
    xc, new_conv = conv1d.conv1d_decode(mixed, conv_state, conv_weight)
    q = xc[:, :Hk * Dk].reshape(B, Hk, 1, Dk)
    k = xc[:, Hk * Dk:2 * Hk * Dk].reshape(B, Hk, 1, Dk)
    v = xc[:, 2 * Hk * Dk:].reshape(B, Hv, 1, Dv)
    a = np.asarray(a, np.float64).reshape(B, Hv, 1)
    b = np.asarray(b, np.float64).reshape(B, Hv, 1)
    o, st = oracle.gdn_serial_gated_f64(q, k, v, a, b, A_log, dt_bias, scale, l2_eps, state,
                                        inplace=inplace)
    y = rmsnorm_gated(o[:, :, 0], np.asarray(z, np.float64).reshape(B, Hv, Dv), norm_weight,
                      norm_eps)
    return y.reshape(B, Hv * Dv), new_conv, st

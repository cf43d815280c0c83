"""Depthwise causal conv1d + SiLU and its window state -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library shares no code with it.

The step that precedes the gated delta rule in the decode block, on its own
page "GDN Conv1D Kernel API Reference":

* prefill (gdn_conv1d_prefill, Parameters and Returns): the raw mixed input
  ``x[B, C, T]`` (q|k|v channels), depthwise weights ``w[C, K]`` (one FIR per
  channel, Notes: groups == C), output silu(causal_conv1d(x)) ``[B, C, T]`` and
  the new window state = the last K RAW tokens ``[B, C, K]`` (introduction).
* decode (gdn_conv1d_decode): one new raw token ``x[B, C]`` and the previous
  window ``state[B, C, K]``; the window shifts by one (oldest dropped, the new
  token appended) and the output is silu of the K-tap dot product of the
  weights with the shifted window (Notes: the FIR reduces to a K-tap dot
  product), which is also the new state.

Readings where the page is silent: the weights are a squeezed depthwise
convolution weight applied as a cross-correlation over the causally padded
input, so w[c, K-1] multiplies the current token and w[c, j] the token
K-1-j steps back; there is no bias; tokens before t = 0 are zero; with T < K
the state's leading entries are zero. silu(y) = y / (1 + e^{-y}).

Everything is evaluated in float64 from the float32 (bf16-exact) inputs.
"""
import numpy as np

__all__ = ["silu", "conv1d_prefill", "conv1d_decode"]


def silu(y):
    """y * sigmoid(y), float64."""
    y = np.asarray(y, dtype=np.float64)
    return y / (1.0 + np.exp(-y))


def conv1d_prefill(x, w):
    """x [B, C, T], w [C, K] -> (out [B, C, T] float64, state [B, C, K] float64).

    y[b, c, t] = sum_j w[c, j] x[b, c, t - (K - 1) + j]   (x = 0 before t = 0)
    out = silu(y); state[b, c, j] = x[b, c, T - K + j]   (0 where T - K + j < 0)
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, C, T = x.shape
    Cw, K = w.shape
    if Cw != C or K < 1:
        raise ValueError("oracle: conv weight must be [C, K], K >= 1")
    y = np.zeros((B, C, T), dtype=np.float64)
    for j in range(K):
        lag = K - 1 - j                       # tap j reads the token `lag` steps back
        if lag >= T:
            continue
        y[:, :, lag:] += w[None, :, j, None] * x[:, :, :T - lag]
    state = np.zeros((B, C, K), dtype=np.float64)
    for j in range(K):
        t = T - K + j
        if t >= 0:
            state[:, :, j] = x[:, :, t]
    return silu(y), state


def conv1d_decode(x, state, w):
    """x [B, C], state [B, C, K], w [C, K] -> (out [B, C], new state [B, C, K]),
    float64: the window drops its oldest token and appends x, then
    out = silu(sum_j w[c, j] window[b, c, j])."""
    x = np.asarray(x, dtype=np.float64)
    state = np.asarray(state, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, C = x.shape
    K = w.shape[1]
    if state.shape != (B, C, K) or w.shape[0] != C:
        raise ValueError("oracle: inconsistent conv decode shapes")
    window = np.concatenate([state[:, :, 1:], x[:, :, None]], axis=2)
    y = np.zeros((B, C), dtype=np.float64)
    for j in range(K):
        y += w[None, :, j] * window[:, :, j]
    return silu(y), window

"""Python binding of libgdn: the gated delta-rule recurrence on MI355X.

Argument marshalling only -- every step of the computation runs in the HIP
kernels of ``libgdn.so`` (built from ``csrc/`` by
``python -m linear_attention_recurrence_chunked_amd.build``). The names
mirror the C ABI in ``include/gdn.h``:

* :func:`chunked_prefill` -> ``gdn_chunked_prefill`` (``gdn_chunked_prefill_inverse``
  when an inverse method is chosen)
* :func:`decode_step`     -> ``gdn_decode_step``
* :func:`chunked_prefill_gated` -> ``gdn_chunked_prefill_gated``
* :func:`decode_step_gated`     -> ``gdn_decode_step_gated``
* :func:`conv1d_prefill`  -> ``gdn_conv1d_prefill``
* :func:`conv1d_decode`   -> ``gdn_conv1d_decode``
* :func:`rmsnorm_gated`   -> ``gdn_rmsnorm_gated``
* :func:`decode_block`    -> ``gdn_decode_block``
* :func:`prefill_workspace_bytes` -> ``gdn_chunked_prefill_workspace_bytes``
* :func:`status_string`   -> ``gdn_status_string``

Tensors are torch tensors on the GPU; torch supplies device memory and the
current stream, nothing else. If ``libgdn.so`` is missing these functions raise
:class:`LibraryNotBuilt`; there is no fallback path.
"""
import ctypes
import os

__all__ = ["chunked_prefill", "decode_step", "chunked_prefill_gated", "decode_step_gated",
           "conv1d_prefill", "conv1d_decode", "rmsnorm_gated", "decode_block",
           "prefill_workspace_bytes", "status_string",
           "GdnError", "LibraryNotBuilt", "load_library", "LIB_PATH", "GDN_F32", "GDN_BF16",
           "GDN_INV_SUBSTITUTION", "GDN_INV_NEUMANN"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_INV_SUBSTITUTION, GDN_INV_NEUMANN = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
          4: "GDN_ERR_DTYPE", 5: "GDN_ERR_ALIGN", 6: "GDN_ERR_ALIAS", 7: "GDN_ERR_WORKSPACE",
          8: "GDN_ERR_HIP", 9: "GDN_ERR_VALUE"}
_F = ctypes.c_float


class LibraryNotBuilt(RuntimeError):
    pass


class GdnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def load_library():
    """Load libgdn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt("%s is not built; run `python -m "
                              "linear_attention_recurrence_chunked_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_chunked_prefill.restype = _I
    lib.gdn_chunked_prefill.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                        _I, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P]
    lib.gdn_chunked_prefill_inverse.restype = _I
    lib.gdn_chunked_prefill_inverse.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                                _I, _I, _I, _I, _I, _I, _I, _I, _P,
                                                ctypes.c_size_t, _P]
    lib.gdn_chunked_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunked_prefill_workspace_bytes.argtypes = [_I] * 7
    lib.gdn_decode_step.restype = _I
    lib.gdn_decode_step.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                    _I, _I, _I, _I, _I, _I, _P]
    lib.gdn_chunked_prefill_gated.restype = _I
    lib.gdn_chunked_prefill_gated.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                              ctypes.c_float, _P, _P, _I, _I, _I, _I, _I, _I,
                                              _I, _P, ctypes.c_size_t, _P]
    lib.gdn_decode_step_gated.restype = _I
    lib.gdn_decode_step_gated.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                          ctypes.c_float, _P, _P, _I, _I, _I, _I, _I, _I, _P]
    lib.gdn_conv1d_prefill.restype = _I
    lib.gdn_conv1d_prefill.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
    lib.gdn_conv1d_decode.restype = _I
    lib.gdn_conv1d_decode.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P]
    lib.gdn_rmsnorm_gated.restype = _I
    lib.gdn_rmsnorm_gated.argtypes = [_P, _P, _P, ctypes.c_float, _P, _I, _I, _I, _I, _I, _P]
    lib.gdn_decode_block.restype = _I
    lib.gdn_decode_block.argtypes = [_P] * 10 + [ctypes.c_float] * 3 + [_P, _P] + [_I] * 7 + [_P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [_I]
    lib.gdn_version.restype = _I
    lib.gdn_version.argtypes = []
    _lib = lib
    return lib


def status_string(code):
    return load_library().gdn_status_string(int(code)).decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v/out must be torch.bfloat16 or torch.float32, got %s" % t.dtype)


def _check(t, name, dtype, device):
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _raise(code):
    if code != 0:
        raise GdnError(code, status_string(code))


def prefill_workspace_bytes(B, Hk, Hv, S, Dk, Dv, dtype_code):
    return int(load_library().gdn_chunked_prefill_workspace_bytes(B, Hk, Hv, S, Dk, Dv,
                                                                  dtype_code))


def chunked_prefill(q, k, v, g_log, beta, scale, state, out=None, workspace=None, stream=None,
                    inverse=None):
    """Chunked gated delta-rule prefill (``gdn_chunked_prefill``).

    q, k [B,Hk,S,Dk] and v [B,Hv,S,Dv] in bf16 or fp32 (one dtype); g_log, beta
    [B,Hv,S] fp32; state [B,Hv,Dk,Dv] fp32, updated in place. Returns out
    [B,Hv,S,Dv] in the compute dtype (allocated if not given). ``inverse``
    (GDN_INV_SUBSTITUTION or GDN_INV_NEUMANN) selects the intra-chunk inverse
    through ``gdn_chunked_prefill_inverse``.
    """
    import torch
    lib = load_library()
    dev = q.device
    code = _dtype_code(q)
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    for t, n in ((g_log, "g_log"), (beta, "beta"), (state, "state")):
        _check(t, n, torch.float32, dev)
    if k.shape != q.shape or v.shape[0] != B or v.shape[2] != S:
        raise ValueError("q/k/v shapes disagree")
    if g_log.shape != (B, Hv, S) or beta.shape != (B, Hv, S) or state.shape != (B, Hv, Dk, Dv):
        raise ValueError("g_log/beta/state shapes disagree with q/v")
    if out is None:
        out = torch.empty((B, Hv, S, Dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", q.dtype, dev)
        if out.shape != (B, Hv, S, Dv):
            raise ValueError("out shape must be [B,Hv,S,Dv]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if inverse is None:
        rc = lib.gdn_chunked_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), g_log.data_ptr(),
                                     beta.data_ptr(), float(scale), state.data_ptr(),
                                     out.data_ptr(), B, Hk, Hv, S, Dk, Dv, code, ws_ptr, ws_bytes,
                                     _stream(stream, dev))
    else:
        rc = lib.gdn_chunked_prefill_inverse(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             g_log.data_ptr(), beta.data_ptr(), float(scale),
                                             state.data_ptr(), out.data_ptr(), B, Hk, Hv, S, Dk,
                                             Dv, code, int(inverse), ws_ptr, ws_bytes,
                                             _stream(stream, dev))
    _raise(rc)
    return out


def decode_step(q, k, v, g_log, beta, scale, state, out=None, stream=None):
    """One-token gated delta-rule step (``gdn_decode_step``), state in place.

    q, k [B,Hk,Dk], v [B,Hv,Dv] (bf16 or fp32); g_log, beta [B,Hv] fp32; state
    [B,Hv,Dk,Dv] fp32. Returns out [B,Hv,Dv].
    """
    import torch
    lib = load_library()
    dev = q.device
    code = _dtype_code(q)
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    for t, n in ((g_log, "g_log"), (beta, "beta"), (state, "state")):
        _check(t, n, torch.float32, dev)
    if k.shape != q.shape or v.shape[0] != B:
        raise ValueError("q/k/v shapes disagree")
    if g_log.shape != (B, Hv) or beta.shape != (B, Hv) or state.shape != (B, Hv, Dk, Dv):
        raise ValueError("g_log/beta/state shapes disagree with q/v")
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", q.dtype, dev)
        if out.shape != (B, Hv, Dv):
            raise ValueError("out shape must be [B,Hv,Dv]")
    rc = lib.gdn_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g_log.data_ptr(),
                             beta.data_ptr(), float(scale), state.data_ptr(), out.data_ptr(),
                             B, Hk, Hv, Dk, Dv, code, _stream(stream, dev))
    _raise(rc)
    return out


def _check_heads(A_log, dt_bias, Hv, dev):
    import torch
    for t, n in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _check(t, n, torch.float32, dev)
        if t.shape != (Hv,):
            raise ValueError("%s must be [Hv]" % n)


def chunked_prefill_gated(q, k, v, a, b, A_log, dt_bias, scale, l2_eps, state, out=None,
                          workspace=None, stream=None):
    """Prefill with the gate and normalisation prologue on the device
    (``gdn_chunked_prefill_gated``).

    q, k [B,Hk,S,Dk] raw (not normalised) and v [B,Hv,S,Dv], bf16 or fp32;
    a, b [B,Hv,S] fp32 gate pre-activations; A_log, dt_bias [Hv] fp32; state
    [B,Hv,Dk,Dv] fp32, updated in place. Returns out [B,Hv,S,Dv].
    """
    import torch
    lib = load_library()
    dev = q.device
    code = _dtype_code(q)
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    for t, n in ((a, "a"), (b, "b"), (state, "state")):
        _check(t, n, torch.float32, dev)
    _check_heads(A_log, dt_bias, Hv, dev)
    if k.shape != q.shape or v.shape[0] != B or v.shape[2] != S:
        raise ValueError("q/k/v shapes disagree")
    if a.shape != (B, Hv, S) or b.shape != (B, Hv, S) or state.shape != (B, Hv, Dk, Dv):
        raise ValueError("a/b/state shapes disagree with q/v")
    if out is None:
        out = torch.empty((B, Hv, S, Dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", q.dtype, dev)
        if out.shape != (B, Hv, S, Dv):
            raise ValueError("out shape must be [B,Hv,S,Dv]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib.gdn_chunked_prefill_gated(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), A_log.data_ptr(),
        dt_bias.data_ptr(), float(scale), float(l2_eps), state.data_ptr(), out.data_ptr(),
        B, Hk, Hv, S, Dk, Dv, code, ws_ptr, ws_bytes, _stream(stream, dev))
    _raise(rc)
    return out


def decode_step_gated(q, k, v, a, b, A_log, dt_bias, scale, l2_eps, state, out=None,
                      stream=None):
    """One-token step with the prologue on the device (``gdn_decode_step_gated``).

    q, k [B,Hk,Dk] raw, v [B,Hv,Dv] (bf16 or fp32); a, b [B,Hv] fp32; A_log,
    dt_bias [Hv] fp32; state [B,Hv,Dk,Dv] fp32, in place. Returns out [B,Hv,Dv].
    """
    import torch
    lib = load_library()
    dev = q.device
    code = _dtype_code(q)
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    for t, n in ((a, "a"), (b, "b"), (state, "state")):
        _check(t, n, torch.float32, dev)
    _check_heads(A_log, dt_bias, Hv, dev)
    if k.shape != q.shape or v.shape[0] != B:
        raise ValueError("q/k/v shapes disagree")
    if a.shape != (B, Hv) or b.shape != (B, Hv) or state.shape != (B, Hv, Dk, Dv):
        raise ValueError("a/b/state shapes disagree with q/v")
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", q.dtype, dev)
        if out.shape != (B, Hv, Dv):
            raise ValueError("out shape must be [B,Hv,Dv]")
    rc = lib.gdn_decode_step_gated(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), A_log.data_ptr(),
        dt_bias.data_ptr(), float(scale), float(l2_eps), state.data_ptr(), out.data_ptr(),
        B, Hk, Hv, Dk, Dv, code, _stream(stream, dev))
    _raise(rc)
    return out


def conv1d_prefill(mixed, weight, out=None, state=None, stream=None):
    """Depthwise causal conv1d + SiLU (``gdn_conv1d_prefill``).

    mixed [B,C,T] bf16 or fp32 (raw q|k|v channels); weight [C,K] fp32,
    K <= 8. Returns (out [B,C,T], state [B,C,K]) in mixed's dtype, allocated
    if not given: out = silu(causal conv), state = the last K raw tokens.
    """
    import torch
    lib = load_library()
    dev = mixed.device
    code = _dtype_code(mixed)
    _check(mixed, "mixed", mixed.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if mixed.dim() != 3 or weight.dim() != 2 or weight.shape[0] != mixed.shape[1]:
        raise ValueError("mixed must be [B,C,T] and weight [C,K]")
    B, C, T = mixed.shape
    K = weight.shape[1]
    if out is None:
        out = torch.empty_like(mixed)
    else:
        _check(out, "out", mixed.dtype, dev)
        if out.shape != mixed.shape:
            raise ValueError("out must be [B,C,T]")
    if state is None:
        state = torch.empty((B, C, K), dtype=mixed.dtype, device=dev)
    else:
        _check(state, "state", mixed.dtype, dev)
        if state.shape != (B, C, K):
            raise ValueError("state must be [B,C,K]")
    _raise(lib.gdn_conv1d_prefill(mixed.data_ptr(), weight.data_ptr(), out.data_ptr(),
                                  state.data_ptr(), B, C, T, K, code, _stream(stream, dev)))
    return out, state


def conv1d_decode(x, state, weight, out=None, stream=None):
    """One conv1d decode token (``gdn_conv1d_decode``): x [B,C] and the window
    state [B,C,K] (updated in place) in bf16 or fp32, weight [C,K] fp32.
    Returns out [B,C]."""
    import torch
    lib = load_library()
    dev = x.device
    code = _dtype_code(x)
    _check(x, "x", x.dtype, dev)
    _check(state, "state", x.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if x.dim() != 2 or weight.dim() != 2 or weight.shape[0] != x.shape[1]:
        raise ValueError("x must be [B,C] and weight [C,K]")
    B, C = x.shape
    K = weight.shape[1]
    if state.shape != (B, C, K):
        raise ValueError("state must be [B,C,K]")
    if out is None:
        out = torch.empty_like(x)
    else:
        _check(out, "out", x.dtype, dev)
        if out.shape != x.shape:
            raise ValueError("out must be [B,C]")
    _raise(lib.gdn_conv1d_decode(x.data_ptr(), weight.data_ptr(), state.data_ptr(),
                                 out.data_ptr(), B, C, K, code, _stream(stream, dev)))
    return out


def rmsnorm_gated(o, z, weight, eps, out=None, stream=None):
    """RMSNormGated epilogue (``gdn_rmsnorm_gated``): o [B,Hv,S,Dv] head-major
    (a prefill output), z [B,S,Hv,Dv] token-major, weight [Dv] fp32. Returns
    out [B,S,Hv,Dv] = o / sqrt(mean(o^2) + eps) * weight * silu(z)."""
    import torch
    lib = load_library()
    dev = o.device
    code = _dtype_code(o)
    _check(o, "o", o.dtype, dev)
    _check(z, "z", o.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if o.dim() != 4:
        raise ValueError("o must be [B,Hv,S,Dv]")
    B, Hv, S, Dv = o.shape
    if z.shape != (B, S, Hv, Dv) or weight.shape != (Dv,):
        raise ValueError("z must be [B,S,Hv,Dv] and weight [Dv]")
    if out is None:
        out = torch.empty_like(z)
    else:
        _check(out, "out", o.dtype, dev)
        if out.shape != z.shape:
            raise ValueError("out must be [B,S,Hv,Dv]")
    _raise(lib.gdn_rmsnorm_gated(o.data_ptr(), z.data_ptr(), weight.data_ptr(), float(eps),
                                 out.data_ptr(), B, Hv, S, Dv, code, _stream(stream, dev)))
    return out


def decode_block(mixed, z, a, b, conv_state_in, conv_weight, A_log, dt_bias, norm_weight,
                 scale, l2_eps, norm_eps, state, Hk, Hv, Dk, Dv, conv_state_out=None,
                 out=None, stream=None):
    """One token through the decode block without projections
    (``gdn_decode_block``). mixed [B,C] (C = 2 Hk Dk + Hv Dv) and z [B,Hv Dv]
    in bf16 or fp32; a, b [B,Hv] fp32; conv_state_in [B,C,K] (compute dtype);
    conv_weight [C,K], A_log, dt_bias [Hv], norm_weight [Dv] fp32; state
    [B,Hv,Dk,Dv] fp32 (in place). Returns (out [B,Hv Dv], conv_state_out)."""
    import torch
    lib = load_library()
    dev = mixed.device
    code = _dtype_code(mixed)
    B, C = mixed.shape
    K = conv_weight.shape[1]
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError("mixed must have 2 Hk Dk + Hv Dv channels")
    for t, n in ((mixed, "mixed"), (z, "z"), (conv_state_in, "conv_state_in")):
        _check(t, n, mixed.dtype, dev)
    for t, n in ((a, "a"), (b, "b"), (conv_weight, "conv_weight"), (A_log, "A_log"),
                 (dt_bias, "dt_bias"), (norm_weight, "norm_weight"), (state, "state")):
        _check(t, n, torch.float32, dev)
    if (z.shape != (B, Hv * Dv) or a.shape != (B, Hv) or b.shape != (B, Hv)
            or conv_state_in.shape != (B, C, K) or conv_weight.shape != (C, K)
            or A_log.shape != (Hv,) or dt_bias.shape != (Hv,) or norm_weight.shape != (Dv,)
            or state.shape != (B, Hv, Dk, Dv)):
        raise ValueError("decode_block: inconsistent shapes")
    if conv_state_out is None:
        conv_state_out = torch.empty_like(conv_state_in)
    else:
        _check(conv_state_out, "conv_state_out", mixed.dtype, dev)
        if conv_state_out.shape != (B, C, K):
            raise ValueError("conv_state_out must be [B,C,K]")
    if out is None:
        out = torch.empty((B, Hv * Dv), dtype=mixed.dtype, device=dev)
    else:
        _check(out, "out", mixed.dtype, dev)
        if out.shape != (B, Hv * Dv):
            raise ValueError("out must be [B,Hv*Dv]")
    _raise(lib.gdn_decode_block(
        mixed.data_ptr(), z.data_ptr(), a.data_ptr(), b.data_ptr(), conv_state_in.data_ptr(),
        conv_state_out.data_ptr(), conv_weight.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
        norm_weight.data_ptr(), float(scale), float(l2_eps), float(norm_eps), state.data_ptr(),
        out.data_ptr(), B, Hk, Hv, Dk, Dv, K, code, _stream(stream, dev)))
    return out, conv_state_out

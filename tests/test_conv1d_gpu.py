"""gdn_conv1d_prefill / gdn_conv1d_decode on the GPU against the fp64 oracle:
every window width K = 1..8, token counts below, at and across the vector
and workgroup boundaries (ragged T), the full conv workload on sampled
channels, chained decode steps at B = 256, and prefill followed by decode.

The window state holds raw tokens, so it must match bit for bit; outputs are
checked with the same relative-error metric and limits as the recurrence."""
import numpy as np
import pytest

from oracle import conv1d as ref
import workloads
from gpu_helpers import check, log, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch_dtype(dtype))


def _weights(w):
    import torch
    return torch.from_numpy(np.ascontiguousarray(w)).cuda()


def _prefill(x, w, dtype):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    out, st = gdn.conv1d_prefill(_dev(x, dtype), _weights(w))
    torch.cuda.synchronize()
    return to_np(out), to_np(st)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8])
def test_conv_prefill_taps(dtype, K):
    for T in (1, 3, 8, 9, 100, 2048, 2055):
        d = workloads.draw_conv(2, 6, T, K, dtype=dtype)
        out, st = _prefill(d["x"], d["w"], dtype)
        ro, rs = ref.conv1d_prefill(d["x"], d["w"])
        log("conv prefill", dtype, "K", K, "T", T)
        check("conv prefill %s K=%d T=%d" % (dtype, K, T), dtype, out, ro, st, rs)
        assert np.array_equal(st, rs), "window state must be the raw tokens exactly"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,C,T", [(3, 40, 6000), (2, 12, 20000), (2, 10, 17001)])
def test_conv_prefill_multi_tile_rows(dtype, B, C, T):
    """Many channels and batches; T = 20000 spreads each row over three
    workgroups (8192 tokens each) with a ragged tail, so the history across
    workgroup boundaries and the window state of the last one are covered
    (T % 8 == 0: the range-checked tile kernel); T = 17001 does the same on
    the general kernel (a last vector only partly inside the row)."""
    d = workloads.draw_conv(B, C, T, 4, dtype=dtype)
    log("conv prefill multi-tile", dtype, B, C, T)
    out, st = _prefill(d["x"], d["w"], dtype)
    ro, rs = ref.conv1d_prefill(d["x"], d["w"])
    check("conv prefill %dx%dx%d %s" % (B, C, T, dtype), dtype, out, ro, st, rs)
    assert np.array_equal(st, rs)


def test_conv_prefill_workload_sampled():
    """The conv workload the bench times (B=4, C=8192, T=8192, K=4, bf16),
    checked against the oracle on 96 sampled channel rows, and the whole
    window state exactly."""
    w = workloads.CONV_WORKLOADS["conv_prefill_b4_t8192"]
    d = workloads.draw_conv(w.B, w.C, w.T, w.K, dtype=w.dtype)
    out, st = _prefill(d["x"], d["w"], w.dtype)
    rng = np.random.default_rng(7)
    rows = rng.choice(w.B * w.C, size=96, replace=False)
    b, c = rows // w.C, rows % w.C
    # each sampled row is its own (1-channel) problem with its channel's weights
    ro = np.stack([ref.conv1d_prefill(d["x"][bi, ci][None, None], d["w"][ci:ci + 1])[0][0, 0]
                   for bi, ci in zip(b, c)])
    rs = d["x"][:, :, w.T - w.K:]
    check("conv workload sampled rows", "bf16", out[b, c], ro, st, rs)
    assert np.array_equal(st, rs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [2, 4, 8])
def test_conv_decode_steps(dtype, K):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_conv(3, 37, 1, K, dtype=dtype, decode=True)
    st_dev = _dev(d["state"], dtype)
    wt = _weights(d["w"])
    st_ref = d["state"].astype(np.float64)
    for step in range(5):
        xs = workloads.draw_conv(3, 37, 1, K, dtype=dtype, step=step + 1, decode=True)["x"]
        o = gdn.conv1d_decode(_dev(xs, dtype), st_dev, wt)
        ro, st_ref = ref.conv1d_decode(xs, st_ref, d["w"])
        torch.cuda.synchronize()
        check("conv decode %s K=%d step %d" % (dtype, K, step), dtype, to_np(o), ro,
              to_np(st_dev), st_ref)
        assert np.array_equal(to_np(st_dev), st_ref)


def test_conv_decode_workload():
    """B=256, C=8192, K=4, bf16, eight chained steps."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    w = workloads.CONV_WORKLOADS["conv_decode_b256"]
    d = workloads.draw_conv(w.B, w.C, 1, w.K, dtype=w.dtype, decode=True)
    st_dev = _dev(d["state"], w.dtype)
    wt = _weights(d["w"])
    st_ref = d["state"].astype(np.float64)
    for step in range(8):
        xs = workloads.draw_conv(w.B, w.C, 1, w.K, dtype=w.dtype, step=step + 1, decode=True)["x"]
        o = gdn.conv1d_decode(_dev(xs, w.dtype), st_dev, wt)
        ro, st_ref = ref.conv1d_decode(xs, st_ref, d["w"])
        torch.cuda.synchronize()
        check("conv decode b256 step %d" % step, "bf16", to_np(o), ro, to_np(st_dev), st_ref)


def test_conv_prefill_then_decode():
    """prefill(T) then decode steps on the GPU match the oracle's prefill of
    the whole sequence."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_conv(2, 24, 300, 4, dtype="bf16")
    x, wv = d["x"], d["w"]
    ro, rs = ref.conv1d_prefill(x, wv)
    o1, st = gdn.conv1d_prefill(_dev(x[:, :, :290], "bf16"), _weights(wv))
    outs = [to_np(o1)]
    for t in range(290, 300):
        outs.append(to_np(gdn.conv1d_decode(_dev(x[:, :, t], "bf16"), st, _weights(wv)))[:, :, None])
    torch.cuda.synchronize()
    check("conv prefill+decode", "bf16", np.concatenate(outs, axis=2), ro, to_np(st), rs)
    assert np.array_equal(to_np(st), rs)

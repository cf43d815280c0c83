"""gdn_chunked_prefill on the GPU against the fp64 oracle, element by element,
on the named workloads at their full sizes and on edge cases (ragged value
slices, padded key dims, GQA ratios, single chunk, weak/strong decay)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check, log, run_prefill, to_np, upload

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _parity(name, d, dtype, scale, inverse=None):
    log("prefill parity:", name, "inverse", inverse,
        {k: v.shape for k, v in d.items() if v is not None})
    out, st = run_prefill(d, dtype, scale, inverse=inverse)
    ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], scale, d["state"])
    return check(name, dtype, out, ro, st, rs)


def test_tiny_f32():
    w = W["tiny_f32"]
    _parity(w.name, workloads.draw_workload(w), "f32", w.scale)


def test_prefill_s2048():
    w = W["prefill_s2048"]
    _parity(w.name, workloads.draw_workload(w), "bf16", w.scale)


def test_prefill_b4_s8192_full():
    """The bench workload, in the launch configuration the bench times."""
    w = W["prefill_b4_s8192"]
    _parity(w.name, workloads.draw_workload(w), "bf16", w.scale)


def test_prefill_b2_s8192_two_strip_slices():
    """B = 2 at the bench's heads and length: the two-strip (32-column)
    slices, element by element over the full 8192 tokens with a carried
    state."""
    w = W["prefill_b4_s8192"]
    d = workloads.draw_prefill(B=2, Hk=16, Hv=32, S=8192, Dk=128, Dv=128, dtype="bf16",
                               state="normal", decay="std", seed=(11, 2, 0))
    _parity("b2 s8192", d, "bf16", w.scale)


@pytest.mark.parametrize("variant", ["std", "strong"])
def test_prefill_s65536(variant):
    w = W["prefill_s65536"]
    _parity("%s/%s" % (w.name, variant), workloads.draw_workload(w, variant=variant), "bf16",
            w.scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_weak_decay(dtype):
    """Slow decay (e^g ~ 0.97): the inverse's off-diagonals and the carry
    across chunks matter for many tokens."""
    w = W["prefill_s2048"]
    d = workloads.draw_prefill(B=1, Hk=4, Hv=8, S=1024, Dk=128, Dv=128, dtype=dtype,
                            state="normal", decay="weak", seed=(1, 2, 0))
    _parity("weak/%s" % dtype, d, dtype, w.scale)


@pytest.mark.parametrize("B,Dv", [(1, 128), (2, 128), (2, 112)])
def test_consumer_pair_slices(B, Dv):
    """Batch x heads too small for four-strip slices (Hv = 32, Dk = 128):
    B = 1 runs one 16-column strip per workgroup, shared by two consumer
    waves that exchange partial products; B = 2 runs two strips per
    workgroup, one consumer wave each, and Dv = 112 leaves the second strip
    of the last slice without columns. Ragged S, a carried state, weak decay
    (the exchange's sums feed every later chunk)."""
    d = workloads.draw_prefill(B=B, Hk=16, Hv=32, S=328, Dk=128, Dv=Dv, dtype="bf16",
                               state="normal", decay="weak", seed=(9, 3, B))
    _parity("pair B=%d Dv=%d" % (B, Dv), d, "bf16", 128 ** -0.5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [
    dict(B=1, Hk=2, Hv=2, S=64, Dk=64, Dv=64),      # one chunk, G = 1
    dict(B=2, Hk=1, Hv=4, S=192, Dk=128, Dv=128),   # G = 4
    dict(B=1, Hk=2, Hv=4, S=256, Dk=80, Dv=48),     # padded Dk, ragged value slice
    dict(B=3, Hk=3, Hv=3, S=128, Dk=16, Dv=112),    # smallest Dk
    dict(B=1, Hk=1, Hv=2, S=320, Dk=128, Dv=16),    # smallest Dv
])
def test_shapes(dtype, shape):
    d = workloads.draw_prefill(dtype=dtype, state="normal", decay="weak", seed=(9, 2, 1), **shape)
    _parity("shape %s %s" % (dtype, shape), d, dtype, 1.0 / np.sqrt(shape["Dk"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_beta_zero_pure_decay(dtype):
    d = workloads.draw_prefill(B=1, Hk=2, Hv=4, S=128, Dk=128, Dv=128, dtype=dtype,
                            state="normal", decay="weak", seed=(9, 2, 2))
    d["beta"][:] = 0.0
    _parity("beta=0 %s" % dtype, d, dtype, 0.5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_state_no_decay(dtype):
    d = workloads.draw_prefill(B=1, Hk=2, Hv=2, S=128, Dk=64, Dv=64, dtype=dtype,
                            state="zero", decay="weak", seed=(9, 2, 3))
    d["g_log"][:] = 0.0
    _parity("g=0 %s" % dtype, d, dtype, 0.125)


def test_split_sequence_carry_is_bitwise():
    """prefill(S1) then prefill(S2) from the carried state equals
    prefill(S1 + S2) bit for bit (chunk boundaries coincide)."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=2, Hk=2, Hv=4, S=384, Dk=128, Dv=128, dtype="bf16",
                            state="normal", decay="weak", seed=(9, 2, 4))
    t = upload(d, "bf16")
    st_full = t["state"].clone()
    o_full = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.1, st_full)
    st = t["state"].clone()
    cut = 128
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1 = gdn.chunked_prefill(sl(t["q"], 0, cut), sl(t["k"], 0, cut), sl(t["v"], 0, cut),
                             sl(t["g_log"], 0, cut), sl(t["beta"], 0, cut), 0.1, st)
    o2 = gdn.chunked_prefill(sl(t["q"], cut, 384), sl(t["k"], cut, 384), sl(t["v"], cut, 384),
                             sl(t["g_log"], cut, 384), sl(t["beta"], cut, 384), 0.1, st)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=2).view(torch.int16), o_full.view(torch.int16))
    assert torch.equal(st, st_full)


def test_deterministic():
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=2, Hk=4, Hv=8, S=512, Dk=128, Dv=128, dtype="bf16",
                            state="normal", seed=(9, 0, 5))
    t = upload(d, "bf16")
    res = []
    for _ in range(2):
        st = t["state"].clone()
        o = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.1, st)
        torch.cuda.synchronize()
        res.append((o.view(torch.int16).clone(), st.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_decode_iterated_matches_prefill():
    """64 decode steps from a state equal one 64-token prefill from it."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=2, Hk=2, Hv=4, S=64, Dk=128, Dv=128, dtype="bf16",
                            state="normal", decay="weak", seed=(9, 2, 6))
    t = upload(d, "bf16")
    st_p = t["state"].clone()
    o_p = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.1, st_p)
    st_d = t["state"].clone()
    outs = []
    for i in range(64):
        outs.append(gdn.decode_step(t["q"][:, :, i].contiguous(), t["k"][:, :, i].contiguous(),
                                    t["v"][:, :, i].contiguous(),
                                    t["g_log"][:, :, i].contiguous(),
                                    t["beta"][:, :, i].contiguous(), 0.1, st_d))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=2)
    ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], 0.1, d["state"])
    check("prefill vs oracle", "bf16", to_np(o_p), ro, to_np(st_p), rs)
    check("decode x64 vs oracle", "bf16", to_np(o_d), ro, to_np(st_d), rs)


def test_error_writes_nothing():
    """An invalid call (Dk = 72, not a multiple of 16) leaves out and state untouched."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=1, Hk=1, Hv=1, S=96, Dk=72, Dv=64, dtype="bf16",
                            state="normal", seed=(9, 0, 7))
    t = upload(d, "bf16")
    out = torch.full((1, 1, 96, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    st = t["state"].clone()
    with pytest.raises(gdn.GdnError) as e:
        gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.1, st, out=out)
    assert e.value.code == 3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.equal(st, t["state"])


# ---------------------------------------------- Neumann-product inverse (A/B)

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_neumann_inverse_workloads(dtype):
    """The Neumann inverse against the oracle on the small fp32 workload and
    the S=2048 bf16 workload (shape and dtype of each), and in weak decay
    where the inverse's off-diagonal entries are largest."""
    import linear_attention_recurrence_chunked_amd as gdn
    w = W["tiny_f32"] if dtype == "f32" else W["prefill_s2048"]
    _parity("neumann " + w.name, workloads.draw_workload(w), w.dtype, w.scale,
            inverse=gdn.GDN_INV_NEUMANN)
    d = workloads.draw_prefill(B=1, Hk=4, Hv=8, S=1024, Dk=128, Dv=128, dtype=dtype,
                            state="normal", decay="weak", seed=(1, 2, 0))
    _parity("neumann weak/%s" % dtype, d, dtype, 1.0 / np.sqrt(128), inverse=gdn.GDN_INV_NEUMANN)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [
    dict(B=1, Hk=2, Hv=2, S=64, Dk=64, Dv=64),
    dict(B=1, Hk=2, Hv=4, S=256, Dk=80, Dv=48),
    dict(B=1, Hk=1, Hv=2, S=320, Dk=128, Dv=16),
])
def test_neumann_inverse_shapes(dtype, shape):
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(dtype=dtype, state="normal", decay="weak", seed=(9, 2, 21), **shape)
    _parity("neumann shape %s %s" % (dtype, shape), d, dtype, 1.0 / np.sqrt(shape["Dk"]),
            inverse=gdn.GDN_INV_NEUMANN)


def test_neumann_matches_substitution():
    """Both inverse methods on the bench workload's shape (B=1 slice): the
    states agree to fp32 rounding, and the bf16 outputs differ by at most one
    bf16 ulp (2^-7 |x|: a rounding flip of the same fp32 result) plus 1e-3 of
    the RMS."""
    import linear_attention_recurrence_chunked_amd as gdn
    from gpu_helpers import rms_err
    w = W["prefill_b4_s8192"]
    d = workloads.draw_workload(w, B=1, S=2048)
    o1, s1 = run_prefill(d, "bf16", w.scale)
    o2, s2 = run_prefill(d, "bf16", w.scale, inverse=gdn.GDN_INV_NEUMANN)
    rms = float(np.sqrt(np.mean(o1.astype(np.float64) ** 2)))
    eo = float(np.max(np.maximum(np.abs(o2 - o1) - 2.0 ** -7 * np.abs(o1), 0.0))) / rms
    es = rms_err(s2, s1)
    log("neumann vs substitution: out %.3e state %.3e" % (eo, es))
    assert eo < 1e-3 and es < 1e-5


# ------------------------------------------------- sequence lengths of any size

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S", [1, 5, 31, 33, 100, 1000])
def test_ragged_sequence_length(dtype, S):
    """A partial last chunk (S not a multiple of the 32-token chunk): exact,
    no output past S, state as the oracle's."""
    d = workloads.draw_prefill(B=2, Hk=2, Hv=4, S=S, Dk=128, Dv=128, dtype=dtype, state="normal",
                            decay="weak", seed=(9, 3, S))
    _parity("ragged S=%d %s" % (S, dtype), d, dtype, 1.0 / np.sqrt(128))


def test_ragged_neumann_and_shapes():
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=1, Hk=2, Hv=4, S=77, Dk=80, Dv=48, dtype="bf16", state="normal",
                            decay="weak", seed=(9, 3, 77))
    _parity("ragged neumann S=77", d, "bf16", 0.1, inverse=gdn.GDN_INV_NEUMANN)
    _parity("ragged S=77 Dk=80 Dv=48", d, "bf16", 0.1)


def test_ragged_out_untouched_past_end():
    """Nothing is written past the last token: out sits at the front of a
    larger buffer filled with a marker, which must survive the call."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=1, Hk=1, Hv=2, S=45, Dk=64, Dv=64, dtype="bf16", state="normal",
                            seed=(9, 3, 45))
    t = upload(d, "bf16")
    n = 1 * 2 * 45 * 64
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:n].view(1, 2, 45, 64)
    gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.1, t["state"], out=out)
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], 0.1, d["state"])
    check("ragged S=45", "bf16", to_np(out), ro, to_np(t["state"]), rs)
    assert torch.all(buf[n:] == 7.0)


def test_ragged_split_carry_matches_oracle():
    """prefill(100) then prefill(284) from the carried state matches the
    oracle over all 384 tokens (chunk boundaries differ from one call of 384)."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d = workloads.draw_prefill(B=2, Hk=2, Hv=4, S=384, Dk=128, Dv=128, dtype="bf16",
                            state="normal", decay="weak", seed=(9, 3, 384))
    t = upload(d, "bf16")
    st = t["state"].clone()
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1 = gdn.chunked_prefill(sl(t["q"], 0, 100), sl(t["k"], 0, 100), sl(t["v"], 0, 100),
                             sl(t["g_log"], 0, 100), sl(t["beta"], 0, 100), 0.1, st)
    o2 = gdn.chunked_prefill(sl(t["q"], 100, 384), sl(t["k"], 100, 384), sl(t["v"], 100, 384),
                             sl(t["g_log"], 100, 384), sl(t["beta"], 100, 384), 0.1, st)
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], 0.1, d["state"])
    check("ragged split 100+284", "bf16", to_np(torch.cat([o1, o2], dim=2)), ro, to_np(st), rs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gqa_equals_repeated_heads(dtype):
    """GQA (Hv = 4 Hk: value head h reads key head h / 4) gives bit for bit
    what the same call gives with q and k repeated per value head (Hk = Hv)."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    G = 4
    d = workloads.draw_prefill(B=2, Hk=2, Hv=2 * G, S=200, Dk=64, Dv=128, dtype=dtype,
                            state="normal", seed=(71, 0, 0))
    dr = dict(d, q=np.repeat(d["q"], G, axis=1), k=np.repeat(d["k"], G, axis=1))
    res = []
    for dd in (d, dr):
        t = upload(dd, dtype)
        o = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], 0.125, t["state"])
        torch.cuda.synchronize()
        res.append((to_np(o), to_np(t["state"])))
    log("GQA vs repeated heads", dtype)
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32))
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))


def test_max_sequence_length_addressing():
    """The longest accepted sequence, S = 4194239, in fp32 at Dk = Dv = 128:
    byte offsets within a stream reach 2,147,483,136 (just below 2^31) and the
    last chunk holds 31 tokens. With beta = 0 and g = 0 the state never
    changes, so out_t = scale S0^T q_t exactly and the final state is S0 bit
    for bit: q is zero except at sampled tokens (the first chunks, tokens
    around the middle, the ragged tail), whose outputs are checked against
    that closed form in fp64, and a few zero-q tokens must give zeros."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    S, D = 4194239, 128
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(4194239)
    sample = np.unique(np.concatenate([np.arange(0, 70), S // 2 + np.arange(-40, 40),
                                       np.arange(S - 100, S), rng.integers(0, S, 60)]))
    zero_q = np.array([100, S // 3, S - 200])
    qs = rng.standard_normal((len(sample), D)).astype(np.float32)
    qs /= np.linalg.norm(qs, axis=1, keepdims=True)
    s0 = (0.02 * rng.standard_normal((D, D))).astype(np.float32)
    q = torch.zeros((1, 1, S, D), dtype=torch.float32, device=dev)
    q[0, 0, torch.from_numpy(sample).to(dev)] = torch.from_numpy(qs).to(dev)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    g = torch.zeros((1, 1, S), dtype=torch.float32, device=dev)
    beta = torch.zeros_like(g)
    state = torch.from_numpy(s0.reshape(1, 1, D, D).copy()).to(dev)
    scale = 1.0 / np.sqrt(D)
    log("max-length prefill: S", S, "fp32, sampled tokens", len(sample))
    out = gdn.chunked_prefill(q, k, v, g, beta, scale, state)
    torch.cuda.synchronize()
    got = out[0, 0, torch.from_numpy(sample).to(dev)].double().cpu().numpy()
    ref = scale * qs.astype(np.float64) @ s0.astype(np.float64)
    err = np.max(np.abs(got - ref) / (np.sqrt(np.mean(ref * ref)) + np.abs(ref)))
    log("max-length prefill: sampled out err %.3e" % err)
    assert err <= 1e-4
    assert torch.count_nonzero(out[0, 0, torch.from_numpy(zero_q).to(dev)]).item() == 0
    assert np.array_equal(state[0, 0].cpu().numpy().view(np.uint32), s0.view(np.uint32))
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_key_overwrite(dtype):
    """g = 0, beta = 1 and orthonormal keys: each step replaces the state's
    component along k_t by v_t, so with q_t = k_t every output is scale v_t
    exactly, whatever the initial state (the delta rule's overwrite property;
    in the chunked form A = 0, T = I and P = scale I)."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    S, D = 96, 128
    rng = np.random.default_rng(96)
    qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    kk = qm[:S].astype(np.float32)                      # S orthonormal rows
    if dtype == "bf16":                                  # exact bf16 keys stay near-orthonormal
        kk = workloads.bf16_round(kk)
    v = rng.standard_normal((1, 1, S, D)).astype(np.float32)
    if dtype == "bf16":
        v = workloads.bf16_round(v)
    d = {"q": kk[None, None].copy(), "k": kk[None, None].copy(), "v": v,
         "g_log": np.zeros((1, 1, S), np.float32), "beta": np.ones((1, 1, S), np.float32),
         "state": (0.5 * rng.standard_normal((1, 1, D, D))).astype(np.float32)}
    t = upload(d, dtype)
    scale = 0.25
    out = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], scale, t["state"])
    torch.cuda.synchronize()
    ref = scale * v.astype(np.float64)
    if dtype == "bf16":
        # bf16 keys are orthonormal only to ~1e-3 (their rounding); the oracle
        # on the same inputs bounds the rounding part
        ro, _ = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], scale, d["state"])
        log("overwrite: oracle vs scale v %.3e" % np.max(np.abs(ro - ref)))
        ref = ro
    err = np.max(np.abs(to_np(out) - ref) / (np.sqrt(np.mean(ref * ref)) + np.abs(ref)))
    log("exact key overwrite %s: out err %.3e" % (dtype, err))
    assert err <= (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("gated", [False, True])
def test_repeat_launches_bitwise_at_bench_size(gated):
    """20 launches of the bench workload (B = 4, Hk = 16, Hv = 32, S = 8192)
    from the same inputs give bitwise the same output and state: a race
    between the waves of a workgroup (the consumers pass the per-chunk
    barrier without waiting for their reads of the next chunk) would show as
    run-to-run differences here."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    from gpu_helpers import upload_raw
    w = W["prefill_b4_s8192"]
    d = workloads.draw_workload(w, raw=True)
    t = upload_raw(d, "bf16") if gated else upload(d, "bf16")
    st0 = t["state"].clone()
    out = torch.empty((w.B, w.Hv, w.S, w.Dv), dtype=torch.bfloat16, device="cuda")
    ref_o = ref_s = None
    for rep in range(20):
        st = st0.clone()
        if gated:
            gdn.chunked_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                      t["dt_bias"], w.scale, 1e-6, st, out=out)
        else:
            gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], w.scale, st,
                                out=out)
        if rep == 0:
            ref_o, ref_s = out.clone(), st.clone()
        else:
            assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), "run %d out" % rep
            assert torch.equal(st.view(torch.int32), ref_s.view(torch.int32)), "run %d state" % rep
    torch.cuda.synchronize()
    log("20 launches bitwise identical, gated" if gated else "20 launches bitwise identical")

"""The entry points under HIP graph capture: a captured sequence of calls
(decode steps, a prefill, decode-block steps) replayed several times, with
eager work and synchronisation between the replays, must reproduce the eager
results bit for bit on every replay. The library records no memset and
allocates nothing, so every call is a plain kernel node."""
import numpy as np
import pytest

import workloads
from gpu_helpers import log, upload

pytestmark = pytest.mark.gpu


def _replays_match(run, reset, outputs, nrep=3):
    """Eager run -> reference; capture; replay nrep times (reset eagerly in
    between) and compare every output tensor bitwise."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(nrep):
        reset()                                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % rep
    log("graph replays match:", nrep)


def test_graph_decode_steps_and_prefill():
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    w = workloads.WORKLOADS["decode_b256"]
    state0, steps = workloads.draw_decode_steps(w, nsteps=6, B=8)
    dev = [upload(d, "bf16") for d in steps]
    st0 = torch.from_numpy(state0).cuda()
    st = st0.clone()
    outs = [torch.empty((8, w.Hv, w.Dv), dtype=torch.bfloat16, device="cuda") for _ in steps]
    pd = workloads.draw_prefill(B=1, Hk=2, Hv=4, S=256, Dk=128, Dv=128, dtype="bf16",
                             state="normal", seed=(9, 0, 30))
    pt = upload(pd, "bf16")
    pst0 = pt["state"].clone()
    pout = torch.empty((1, 4, 256, 128), dtype=torch.bfloat16, device="cuda")

    def reset():
        st.copy_(st0)
        pt["state"].copy_(pst0)

    def run():
        for t, o in zip(dev, outs):
            gdn.decode_step(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                            t["g_log"][:, :, 0], t["beta"][:, :, 0], w.scale, st, out=o)
        gdn.chunked_prefill(pt["q"], pt["k"], pt["v"], pt["g_log"], pt["beta"], 0.1,
                            pt["state"], out=pout)

    for t in dev:   # the per-step slices must be contiguous before capture
        for k in ("q", "k", "v", "g_log", "beta"):
            t[k] = t[k][:, :, :1].contiguous()
    _replays_match(run, reset, outs + [st, pout, pt["state"]])


def test_graph_decode_block():
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    B, Hk, Hv, Dk, Dv, K = 4, 2, 4, 128, 128, 4
    d0 = workloads.draw_block(B, Hk, Hv, Dk, Dv, K)
    up = lambda a, bf: torch.from_numpy(a).cuda().to(torch.bfloat16 if bf else torch.float32)
    toks = [d0] + [workloads.draw_block(B, Hk, Hv, Dk, Dv, K, step=i, with_state=False)
                   for i in (1, 2, 3)]
    dt = [{k: up(t[k], k in ("mixed", "z")) for k in ("mixed", "z", "a", "b")} for t in toks]
    fx = {k: up(d0[k], False) for k in ("conv_weight", "A_log", "dt_bias", "norm_weight")}
    st0, cs0 = up(d0["state"], False), up(d0["conv_state"], True)
    st, win = st0.clone(), [cs0.clone(), torch.empty_like(cs0)]
    outs = [torch.empty((B, Hv * Dv), dtype=torch.bfloat16, device="cuda") for _ in toks]

    def reset():
        st.copy_(st0)
        win[0].copy_(cs0)

    def run():
        for i, t in enumerate(dt):
            gdn.decode_block(t["mixed"], t["z"], t["a"], t["b"], win[i & 1], fx["conv_weight"],
                             fx["A_log"], fx["dt_bias"], fx["norm_weight"], 0.1, 1e-6, 1e-5, st,
                             Hk, Hv, Dk, Dv, conv_state_out=win[(i + 1) & 1], out=outs[i])

    _replays_match(run, reset, outs + [st, win[0]])

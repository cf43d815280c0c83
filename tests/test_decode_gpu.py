"""gdn_decode_step on the GPU against the fp64 oracle (token-serial recurrence
with S = 1, state carried across steps)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check, log, to_np, upload, TOL

pytestmark = pytest.mark.gpu


def _run_steps(w, nsteps, dtype=None, **over):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    dtype = dtype or w.dtype
    state0, steps = workloads.draw_decode_steps(w, nsteps=nsteps, **over)
    st_dev = torch.from_numpy(state0).cuda()
    st_ref = state0.astype(np.float64)
    outs, refs = [], []
    for d in steps:
        t = upload(d, dtype)
        # decode layout: drop the S = 1 axis
        o = gdn.decode_step(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                            t["g_log"][:, :, 0].contiguous(), t["beta"][:, :, 0].contiguous(),
                            w.scale, st_dev)
        outs.append(to_np(o))
        ro, st_ref = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], w.scale,
                                       st_ref, inplace=True)
        refs.append(ro[:, :, 0])
    torch.cuda.synchronize()
    return np.stack(outs), np.stack(refs), to_np(st_dev), st_ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [dict(B=3, Hk=2, Hv=4, Dk=128, Dv=128),
                                   dict(B=2, Hk=1, Hv=3, Dk=64, Dv=32),
                                   dict(B=2, Hk=2, Hv=2, Dk=48, Dv=80)])
def test_decode_small(dtype, shape):
    w = workloads.WORKLOADS["decode_b256"]
    log("decode small", dtype, shape)
    o, ro, s, rs = _run_steps(w, 8, dtype=dtype, **shape)
    check("decode %s %s" % (dtype, shape), dtype, o, ro, s, rs)


def test_decode_b256_64_steps():
    """The full decode workload: B=256, Hk=16, Hv=32, Dk=Dv=128, 64 steps."""
    w = workloads.WORKLOADS["decode_b256"]
    log("decode_b256 x 64 steps")
    o, ro, s, rs = _run_steps(w, w.steps)
    check("decode_b256 64 steps", "bf16", o, ro, s, rs)


def test_decode_deterministic():
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    w = workloads.WORKLOADS["decode_b256"]
    state0, steps = workloads.draw_decode_steps(w, nsteps=2, B=8)
    res = []
    for _ in range(2):
        st = torch.from_numpy(state0).cuda()
        outs = []
        for d in steps:
            t = upload(d, "bf16")
            outs.append(gdn.decode_step(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                                        t["g_log"][:, :, 0].contiguous(),
                                        t["beta"][:, :, 0].contiguous(), w.scale, st))
        torch.cuda.synchronize()
        res.append((torch.stack(outs).view(torch.int16).cpu(), st.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_decode_gqa_equals_repeated_heads():
    """GQA (Hv = 2 Hk) gives bit for bit what the same step gives with q and k
    repeated per value head (Hk = Hv)."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    w = workloads.WORKLOADS["decode_b256"]
    state0, steps = workloads.draw_decode_steps(w, nsteps=1, B=8, Hk=4, Hv=8)
    d = steps[0]
    dr = dict(d, q=np.repeat(d["q"], 2, axis=1), k=np.repeat(d["k"], 2, axis=1))
    res = []
    for dd in (d, dr):
        t = upload(dd, "bf16")
        st = torch.from_numpy(state0).cuda()
        o = gdn.decode_step(t["q"][:, :, 0].contiguous(), t["k"][:, :, 0].contiguous(),
                            t["v"][:, :, 0].contiguous(), t["g_log"][:, :, 0].contiguous(),
                            t["beta"][:, :, 0].contiguous(), w.scale, st)
        torch.cuda.synchronize()
        res.append((to_np(o), to_np(st)))
    log("decode GQA vs repeated heads")
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32))
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))

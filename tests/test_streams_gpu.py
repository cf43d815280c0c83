"""Calls on several HIP streams at once. The library keeps no state between
calls, so independent problems launched on different streams without any
synchronisation between them must give, bit for bit, what each gives alone
on one stream (and the oracle's result to the usual tolerance)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check, log, to_np, upload

pytestmark = pytest.mark.gpu


def test_concurrent_streams_match_serial():
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    shapes = [dict(B=2, Hk=2, Hv=4, S=500, Dk=128, Dv=128), dict(B=1, Hk=3, Hv=6, S=333, Dk=64, Dv=96)]
    draws = [workloads.draw_prefill(dtype="bf16", state="normal", seed=(61, i, 0), **sh)
             for i, sh in enumerate(shapes)]
    w = workloads.WORKLOADS["decode_b256"]
    state0, steps = workloads.draw_decode_steps(w, nsteps=4, B=16)

    def launch(stream_of):
        """Two prefills and four decode steps, each problem on its own stream."""
        res = []
        for i, d in enumerate(draws):
            with torch.cuda.stream(stream_of(i)):
                t = upload(d, "bf16")
                out = gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"],
                                          1.0 / np.sqrt(d["q"].shape[-1]), t["state"])
                res.append((out, t["state"]))
        with torch.cuda.stream(stream_of(len(draws))):
            st = torch.from_numpy(state0).cuda()
            outs = []
            for s in steps:
                t = upload(s, "bf16")
                outs.append(gdn.decode_step(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                                            t["g_log"][:, :, 0].contiguous(),
                                            t["beta"][:, :, 0].contiguous(), w.scale, st))
            res.append((torch.stack(outs), st))
        return res

    default = torch.cuda.current_stream()
    serial = launch(lambda i: default)
    torch.cuda.synchronize()
    serial = [(to_np(o), to_np(s)) for o, s in serial]
    streams = [torch.cuda.Stream() for _ in range(len(draws) + 1)]
    for s in streams:
        s.wait_stream(default)
    concurrent = launch(lambda i: streams[i])
    torch.cuda.synchronize()
    for k, ((o1, s1), (o2, s2)) in enumerate(zip(serial, concurrent)):
        assert np.array_equal(o1.view(np.uint8), to_np(o2).view(np.uint8)), "problem %d out" % k
        assert np.array_equal(s1.view(np.uint8), to_np(s2).view(np.uint8)), "problem %d state" % k
    for i, d in enumerate(draws):
        ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"],
                                   1.0 / np.sqrt(d["q"].shape[-1]), d["state"])
        check("stream prefill %d" % i, "bf16", serial[i][0], ro, serial[i][1], rs)
    log("concurrent streams: %d problems bitwise equal to one-stream runs" % len(serial))

"""Seeded random-shape sweep of the prefill and decode entry points against
the fp64 oracle: batch, key heads, GQA ratio, sequence length (ragged
included), head dims (multiples of 16 up to 128), dtype, decay regime,
inverse method and the gated prologue drawn per case. Deterministic: the
cases come from a fixed seed, and each prints its parameters first."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check, log, run_prefill, to_np, upload, upload_raw

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(2024)
CASES = []
for _ in range(24):
    CASES.append(dict(B=int(_R.integers(1, 4)), Hk=int(_R.integers(1, 4)),
                      G=int(_R.choice([1, 2, 4])), S=int(_R.choice([1, 17, 32, 64, 95, 200, 333])),
                      Dk=int(16 * _R.integers(1, 9)), Dv=int(16 * _R.integers(1, 9)),
                      dtype=str(_R.choice(["bf16", "f32"])),
                      decay=str(_R.choice(["std", "weak", "strong"])),
                      neumann=bool(_R.random() < 0.25), gated=bool(_R.random() < 0.3)))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_sweep(case):
    import linear_attention_recurrence_chunked_amd as gdn
    c = CASES[case]
    log("sweep case", case, c)
    d = workloads.draw_prefill(B=c["B"], Hk=c["Hk"], Hv=c["Hk"] * c["G"], S=c["S"], Dk=c["Dk"],
                            Dv=c["Dv"], dtype=c["dtype"], state="normal", decay=c["decay"],
                            seed=(50, case, 0), raw=c["gated"])
    scale = 1.0 / np.sqrt(c["Dk"])
    if c["gated"]:
        import torch
        t = upload_raw(d, c["dtype"])
        out = gdn.chunked_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                        t["dt_bias"], scale, 1e-6, t["state"])
        torch.cuda.synchronize()
        o, st = to_np(out), to_np(t["state"])
        ro, rs = oracle.gdn_serial_gated(d["q_raw"], d["k_raw"], d["v"], d["a"], d["b"],
                                         d["A_log"], d["dt_bias"], scale, 1e-6, d["state"])
    else:
        o, st = run_prefill(d, c["dtype"], scale,
                            inverse=gdn.GDN_INV_NEUMANN if c["neumann"] else None)
        ro, rs = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], scale,
                                   d["state"])
    check("sweep %d" % case, c["dtype"], o, ro, st, rs)


@pytest.mark.parametrize("case", range(8))
def test_decode_sweep(case):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    c = CASES[case]
    log("decode sweep case", case, c)
    w = workloads.WORKLOADS["decode_b256"]
    state0, steps = workloads.draw_decode_steps(w, nsteps=3, B=c["B"], Hk=c["Hk"],
                                             Hv=c["Hk"] * c["G"], Dk=c["Dk"], Dv=c["Dv"])
    st = torch.from_numpy(state0).cuda()
    st_ref = state0.astype(np.float64)
    scale = 1.0 / np.sqrt(c["Dk"])
    outs, refs = [], []
    for d in steps:
        t = upload(d, c["dtype"])
        outs.append(to_np(gdn.decode_step(t["q"][:, :, 0], t["k"][:, :, 0], t["v"][:, :, 0],
                                          t["g_log"][:, :, 0].contiguous(),
                                          t["beta"][:, :, 0].contiguous(), scale, st)))
        ro, st_ref = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], scale,
                                       st_ref, inplace=True)
        refs.append(ro[:, :, 0])
    torch.cuda.synchronize()
    check("decode sweep %d" % case, c["dtype"], np.stack(outs), np.stack(refs), to_np(st),
          st_ref)

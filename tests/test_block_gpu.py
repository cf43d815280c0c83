"""gdn_rmsnorm_gated and gdn_decode_block on the GPU against the fp64 oracle:
the norm on several head sizes and on sampled rows of the full prefill
output; the fused decode block on small shapes (both dtypes, conv widths 3
and 4, GQA) and at B = 256 over chained steps, with the conv windows checked
bit for bit."""
import numpy as np
import pytest

from oracle import block as ref
import workloads
from gpu_helpers import TOL, check, log, out_err, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch_dtype(dtype)) if dtype else t


def _round(x, dtype):
    return workloads.bf16_round(x) if dtype == "bf16" else np.asarray(x, np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Dv", [16, 48, 64, 128])
@pytest.mark.parametrize("B,Hv,S", [(2, 3, 37), (1, 8, 37)])
def test_rmsnorm_gated(dtype, Dv, B, Hv, S):
    """Hv = 3: one head per tile; Hv = 8: tiles of four heads. S = 37 leaves
    a partial token tile either way."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    r = np.random.default_rng([300, Dv, Hv])
    o = _round(r.standard_normal((B, Hv, S, Dv)).astype(np.float32) * 3.0, dtype)
    z = _round(r.standard_normal((B, S, Hv, Dv)).astype(np.float32), dtype)
    w = (1.0 + 0.1 * r.standard_normal(Dv)).astype(np.float32)
    y = gdn.rmsnorm_gated(_dev(o, dtype), _dev(z, dtype), _dev(w), 1e-5)
    torch.cuda.synchronize()
    ry = ref.rmsnorm_gated(np.transpose(o, (0, 2, 1, 3)), z, w, 1e-5)
    e = out_err(to_np(y), ry, dtype)
    log("rmsnorm", dtype, Dv, B, Hv, S, "err %.3e" % e)
    assert e <= TOL[dtype]["out"], e


def test_rmsnorm_gated_prefill_output_sampled():
    """The full bench prefill output shape (B=4, Hv=32, S=8192, Dv=128, bf16),
    4096 sampled (token, head) rows against the oracle."""
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    B, Hv, S, Dv = 4, 32, 8192, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    o = (torch.randn((B, Hv, S, Dv), device="cuda", generator=g) * 2).to(torch.bfloat16)
    z = torch.randn((B, S, Hv, Dv), device="cuda", generator=g).to(torch.bfloat16)
    w = 1.0 + 0.1 * torch.randn((Dv,), device="cuda", generator=g)
    y = gdn.rmsnorm_gated(o, z, w, 1e-6)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    b, s, h = rng.integers(0, B, 4096), rng.integers(0, S, 4096), rng.integers(0, Hv, 4096)
    on, zn, yn = to_np(o), to_np(z), to_np(y)
    ry = ref.rmsnorm_gated(on[b, h, s], zn[b, s, h], to_np(w), 1e-6)
    e = out_err(yn[b, s, h], ry, "bf16")
    log("rmsnorm full-size sampled err %.3e" % e)
    assert e <= TOL["bf16"]["out"], e


def _block_steps(B, Hk, Hv, Dk, Dv, K, dtype, nsteps):
    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    d0 = workloads.draw_block(B, Hk, Hv, Dk, Dv, K, dtype=dtype)
    cin = _dev(d0["conv_state"], dtype)
    cout = torch.empty_like(cin)
    st = _dev(d0["state"])
    fixed = {k: _dev(d0[k]) for k in ("conv_weight", "A_log", "dt_bias", "norm_weight")}
    conv_ref, st_ref = d0["conv_state"], d0["state"].astype(np.float64)
    res = []
    for step in range(nsteps):
        d = d0 if step == 0 else workloads.draw_block(B, Hk, Hv, Dk, Dv, K, dtype=dtype, step=step,
                                                    with_state=False)
        y, _ = gdn.decode_block(_dev(d["mixed"], dtype), _dev(d["z"], dtype), _dev(d["a"]),
                                _dev(d["b"]), cin, fixed["conv_weight"], fixed["A_log"],
                                fixed["dt_bias"], fixed["norm_weight"], 0.1, 1e-6, 1e-5, st,
                                Hk, Hv, Dk, Dv, conv_state_out=cout)
        ry, conv_ref, st_ref = ref.decode_block(d["mixed"], d["z"], d["a"], d["b"], conv_ref,
                                                d0["conv_weight"], d0["A_log"], d0["dt_bias"],
                                                d0["norm_weight"], st_ref, 0.1, 1e-6, 1e-5,
                                                Hk, Hv, Dk, Dv)
        torch.cuda.synchronize()
        res.append((to_np(y), ry, to_np(st), st_ref.copy(), to_np(cout), conv_ref.copy()))
        cin, cout = cout, cin                   # the new windows feed the next step
    return res


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [dict(B=3, Hk=2, Hv=4, Dk=128, Dv=128, K=4),
                                   dict(B=2, Hk=1, Hv=3, Dk=64, Dv=32, K=3),
                                   dict(B=2, Hk=2, Hv=2, Dk=48, Dv=80, K=2)])
def test_decode_block_small(dtype, shape):
    log("decode block", dtype, shape)
    for i, (y, ry, st, rs, cw, rcw) in enumerate(_block_steps(dtype=dtype, nsteps=4, **shape)):
        check("block %s %s step %d" % (dtype, shape, i), dtype, y, ry, st, rs)
        assert np.array_equal(cw, rcw), "conv windows must be the raw tokens exactly"


def test_decode_block_b256():
    """B=256, Hk=16, Hv=32, Dk=Dv=128, K=4, bf16, four chained steps."""
    log("decode block B=256")
    for i, (y, ry, st, rs, cw, rcw) in enumerate(
            _block_steps(256, 16, 32, 128, 128, 4, "bf16", 4)):
        check("block b256 step %d" % i, "bf16", y, ry, st, rs)
        assert np.array_equal(cw, rcw)

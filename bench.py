"""Benchmark of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only prefill|decode|prefill_gated|decode_gated|conv_prefill|
                            conv_decode|rmsnorm|decode_block|inverse_ab|copy]

One step = one ``gdn_chunked_prefill`` call on the batched long prefill
workload (B=4, Hk=16, Hv=32, Dk=Dv=128, S=8192, bf16 q/k/v, fp32 g/beta and
state, state carried in place from step to step). All inputs are seeded,
synthetic and resident in HBM before timing starts. W untimed warm-up steps
and a settling phase (further calls until the device has been busy for at
least 300 ms: the GPU needs ~100 ms of load to reach its steady clocks, and
the host-side input draws between sections let them drop), then exactly K
timed steps bracketed by device synchronisation; each launch is also
bracketed by HIP events on the launch stream to get the kernel's own duration
for the roofline. The shader clock (amdsmi) is sampled during the headline's
settling phase and reported under "sclk".

The decode path (B=256 single-token steps, 64 autoregressive steps with fresh
inputs) is measured the same way in the same run -- K/10 timed passes of 64
steps -- and reported under "decode".

The gated entry points (gate and L2-norm prologue on the device, raw q/k and
gate pre-activations as inputs) are timed the same way on the same workloads
and reported under "prefill_gated" and "decode_gated"; the single-sequence
prefill workloads (B=1: S=2048 from a zero state; S=65536 from a carried
state, standard and strong decay) under "prefill_s2048" and
"prefill_s65536"; the depthwise conv1d that precedes the recurrence (prefill
over the B=4, T=8192 mixed q|k|v tensor with C = 8192 channels and K = 4
taps; one decode token at B=256) under "conv1d_prefill" and "conv1d_decode";
the RMSNormGated epilogue over the prefill output under "rmsnorm_gated"; the
fused decode block (conv1d step, prologue, recurrence, RMSNormGated; B=256,
K=4) under "decode_block". The conv1d decode call lasts less than the host's
launch gap; its kernel time comes from 10 calls captured in a HIP graph and
replayed back to back.

Last, "inverse_ab" times the prefill with each intra-chunk inverse (blocked
substitution, the default, and the Neumann product) at S = 128 .. 8192 with
the other shapes of the headline workload at batch 2 (other kernel instances
than the headline's, so that a profiler's per-kernel statistics of the run
keep them apart): the shape of the pages' only measured comparison between
inverse methods.

``--only copy`` runs a plain device-to-device copy of ``--copy-mib`` MiB
(used to calibrate the HBM byte counters of rocprofv3 against a kernel of
known traffic); ``--only <section>`` runs one section alone.

Roofline (per launch, algorithmic, see the workload docstrings below):
* prefill: HBM bytes = tokens x (q + k + v + out + g + beta) + state in/out;
  algorithmic MFMA flops (a fixed count of the method's work at 64-token
  chunks, 4.24 MFLOP per token on the headline shapes) reported as
  "mfma_util" against the bf16 dense peak, the same count at the kernel's own
  32-token chunks beside it, and under "mfma_util.counter" the issued bf16
  MFMA flops that rocprofv3 counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512,
  committed summary) over this run's launch time, with the MFMA busy fraction
  and shader clock measured with them.
* decode: HBM bytes = 2 x fp32 state + q, k, v, out, g, beta.
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "GDN prefill tokens/s + MFMA util (S=8192); decode steps/s + HBM GB/s"


def prefill_algorithmic(B, Hk, Hv, S, Dk, Dv, esize=2, chunk=64):
    """Algorithmic HBM bytes and MFMA flops of one prefill call.

    bytes: q, k [B,Hk,S,Dk] + v, out [B,Hv,S,Dv] in the operand type, g and
    beta fp32 [B,Hv,S], the fp32 state read once and written once.
    flops (per value head and chunk of C tokens; lower-triangular products
    counted at half size; K K^T and Q K^T shared inside a GQA group):
      W = T K and U~ = T V: C^2 (Dk + Dv); W S, Q S, K^T U: 3 x 2 C Dk Dv;
      P U: C^2 Dv; T: C^3 / 3; per key head: K K^T, Q K^T: 2 x C^2 Dk.
    The reported utilisation uses C = 64, a fixed count of the method's work
    (4.24 MFLOP per token at Hk=16, Hv=32, Dk=Dv=128) that does not depend on
    the kernel's own chunk length (32, whose count is reported beside it).
    """
    tokens = B * S
    nbytes = (tokens * (2 * Hk * Dk + 2 * Hv * Dv) * esize + tokens * Hv * 8
              + 2 * B * Hv * Dk * Dv * 4)
    C = chunk
    per_chunk_vh = C * C * (Dk + Dv) + 6 * C * Dk * Dv + C * C * Dv + C ** 3 / 3.0
    per_chunk_kh = 2 * C * C * Dk
    nchunks = B * S / C
    flops = nchunks * (Hv * per_chunk_vh + Hk * per_chunk_kh)
    return float(nbytes), float(flops)


KERNEL_CHUNK = 32              # the prefill kernel's own chunk length


def decode_algorithmic(B, Hk, Hv, Dk, Dv, esize=2):
    """HBM bytes of one decode step: fp32 state read + write, q, k, v, out, g, beta."""
    return float(2 * B * Hv * Dk * Dv * 4 + (2 * B * Hk * Dk + 2 * B * Hv * Dv) * esize
                 + B * Hv * 8)


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "gdn_prefill_kernel": "linear_attention_recurrence_chunked_amd/csrc/gdn_prefill.hip",
    "gdn_decode_kernel": "linear_attention_recurrence_chunked_amd/csrc/gdn_decode.hip",
}
KERNEL_SOURCES["gdn_prefill_kernel_gated"] = KERNEL_SOURCES["gdn_prefill_kernel"]
KERNEL_SOURCES["gdn_decode_kernel_gated"] = KERNEL_SOURCES["gdn_decode_kernel"]
KERNEL_SOURCES["gdn_conv1d_prefill_tile_kernel"] = "linear_attention_recurrence_chunked_amd/csrc/gdn_conv1d.hip"
KERNEL_SOURCES["gdn_conv1d_decode_kernel"] = KERNEL_SOURCES["gdn_conv1d_prefill_tile_kernel"]
KERNEL_SOURCES["gdn_rmsnorm_gated_kernel"] = "linear_attention_recurrence_chunked_amd/csrc/gdn_norm.hip"
KERNEL_SOURCES["gdn_decode_kernel_block"] = KERNEL_SOURCES["gdn_decode_kernel"]


def source_digest(kernel):
    """Digest of a kernel source's code: comments and whitespace are left
    out, so that a comment edit does not void the counters taken for it.
    (The sources hold no string literal with a comment marker.)"""
    import hashlib
    import re
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel])) as f:
        text = f.read()
    code = re.sub(r"/\*.*?\*/|//[^\n]*", "", text, flags=re.S)
    return hashlib.sha256("".join(code.split()).encode()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def mfma_counters(kernel, kern_ms):
    """Counter-based MFMA utilisation of a prefill kernel: the issued bf16
    MFMA flops per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) from the
    committed rocprofv3 summary over this run's launch time, the MFMA busy
    fraction and the shader clock measured with them; None when the kernel
    source changed since the counters were taken."""
    path = os.path.join(PROFILES, "mfma_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(kernel):
        return None
    issued = rec["issued_bf16_flops_per_launch"] / (kern_ms / 1e3) / 1e12
    return {"issued_bf16_tflops": issued, "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": issued / BF16_PEAK_TFLOPS,
            "issued_bf16_flops_per_launch": rec["issued_bf16_flops_per_launch"],
            "mfma_busy_fraction": rec["mfma_busy_fraction"], "sclk_ghz": rec["sclk_ghz"],
            "source": "profiles/mfma_counters.json"}


def mfma_util(flops, kern_ms, w, counter=None):
    """Algorithmic MFMA utilisation of a prefill launch against the bf16 dense
    peak (the fixed 64-token count), with the kernel's own 32-token count and
    the counter-based issue rate beside it."""
    kflops = prefill_algorithmic(w.B, w.Hk, w.Hv, w.S, w.Dk, w.Dv, chunk=KERNEL_CHUNK)[1]
    rate = lambda f: f / (kern_ms / 1e3) / 1e12
    return {"achieved_tflops": rate(flops), "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": rate(flops) / BF16_PEAK_TFLOPS,
            "algorithmic_flops_per_launch": flops,
            "flops_per_token": flops / (w.B * w.S),
            "count": "chunk length 64, triangles at half size, K K^T and Q K^T once per key head",
            "kernel_chunk32": {"flops_per_launch": kflops, "frac": rate(kflops) / BF16_PEAK_TFLOPS,
                               "note": "the same count at the kernel's own 32-token chunks"},
            "counter": counter}


def clock_record(clocks):
    """The shader clock samples taken while the headline prefill settled."""
    if not clocks:
        return None
    c = np.asarray(clocks, dtype=np.float64)
    return {"median_mhz": float(np.median(c)), "min_mhz": float(c.min()),
            "max_mhz": float(c.max()), "samples": int(c.size),
            "source": "amdsmi current gfx clock (torch.cuda.clock_rate), sampled between "
                      "batches of the settling calls right before the timed prefill calls"}


def long_section(row, hbm):
    """Bench-line section of a single-sequence prefill workload."""
    wl, lms, lkern, lbytes, lflops = row
    tokens = wl.B * wl.S
    return {"workload": wl.name, "B": wl.B, "Hk": wl.Hk, "Hv": wl.Hv, "S": wl.S, "Dk": wl.Dk,
            "Dv": wl.Dv, "state": "zero" if wl.state == "zero" else "N(0, 0.02^2), carried",
            "value": tokens / (lms / 1e3), "unit": "tokens/s", "ms_per_step": lms,
            "roofline": dict(bound="hbm", kernel="gdn_prefill_kernel (B=1 instance)",
                             traffic=None, **hbm(lbytes, lkern)),
            "mfma_util": mfma_util(lflops, lkern, wl)}


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


L2_EPS = 1e-6                  # epsilon of the gated entry points' q/k normalisation
SETTLE_MS = 300.0              # minimum busy time before each timed region


def progress(msg):
    """One line on stderr per finished section (the JSON line goes to stdout)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def _clock_mhz(torch):
    """Current shader (gfx) clock of device 0 in MHz as amdsmi reports it, or
    None where that query is unavailable."""
    try:
        return float(torch.cuda.clock_rate(0))
    except Exception:
        return None


def settle(torch, step, warmup, min_ms=SETTLE_MS, clocks=None):
    """The W warm-up calls, then further calls until the device has been busy
    for at least ``min_ms`` of wall time: the GPU needs ~100 ms of load to
    reach its steady clocks, and the host work between timed sections (input
    draws) lets them drop again. With ``clocks`` (a list), the shader clock is
    sampled between batches of calls and appended. Returns the number of calls."""
    for i in range(warmup):
        step(i)
    n = warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:
        for i in range(8):
            step(i)
        n += 8
        if clocks is not None:
            c = _clock_mhz(torch)
            if c is not None:
                clocks.append(c)
        # synchronised per batch, so that the time counted is the device's
        # (the host would otherwise queue far more calls than it waits for)
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n




def bench_prefill(torch, gdn, w, d, steps, warmup, gated=False, clocks=None):
    """Times the prefill on the draw ``d`` (ungated: normalised q/k, g_log,
    beta; gated: the raw q/k, a, b, A_log, dt_bias of the same draw) with the
    shapes of ``w``; the state is carried from call to call."""
    dev = torch.device("cuda", 0)
    keys = (("q_raw", "k_raw", "v", "a", "b", "A_log", "dt_bias") if gated
            else ("q", "k", "v", "g_log", "beta"))
    t = {k: torch.from_numpy(d[k]).to(dev) for k in keys}
    for k in keys[:3]:
        t[k] = t[k].to(torch.bfloat16)
    state = torch.from_numpy(d["state"]).to(dev)
    out = torch.empty((w.B, w.Hv, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i=0):
        if gated:
            gdn.chunked_prefill_gated(t["q_raw"], t["k_raw"], t["v"], t["a"], t["b"], t["A_log"],
                                      t["dt_bias"], w.scale, L2_EPS, state, out=out,
                                      stream=stream)
        else:
            gdn.chunked_prefill(t["q"], t["k"], t["v"], t["g_log"], t["beta"], w.scale, state,
                                out=out, stream=stream)

    settle(torch, step, warmup, clocks=clocks)
    ev = _events(torch, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_step = (t1 - t0) * 1e3 / steps
    nbytes, flops = prefill_algorithmic(w.B, w.Hk, w.Hv, w.S, w.Dk, w.Dv)
    return ms_step, kern_ms, nbytes, flops


def bench_decode(torch, gdn, w, state0, steps, reps, warmup, gated=False):
    """Times ``reps`` passes over the decode steps (each a dict of one token's
    inputs, drawn with ``raw=True``), state carried on the device."""
    dev = torch.device("cuda", 0)
    st = torch.from_numpy(state0).to(dev)
    tok = lambda s, k: torch.from_numpy(np.ascontiguousarray(s[k][:, :, 0])).to(dev)
    dev_steps = []
    for s in steps:
        if gated:
            dev_steps.append({"q": tok(s, "q_raw").to(torch.bfloat16),
                              "k": tok(s, "k_raw").to(torch.bfloat16),
                              "v": tok(s, "v").to(torch.bfloat16),
                              "g": tok(s, "a"), "b": tok(s, "b"),
                              "A_log": torch.from_numpy(s["A_log"]).to(dev),
                              "dt_bias": torch.from_numpy(s["dt_bias"]).to(dev)})
        else:
            dev_steps.append({"q": tok(s, "q").to(torch.bfloat16),
                              "k": tok(s, "k").to(torch.bfloat16),
                              "v": tok(s, "v").to(torch.bfloat16),
                              "g": tok(s, "g_log"), "b": tok(s, "beta")})
    out = torch.empty((w.B, w.Hv, w.Dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run64(evs=None):
        stream = torch.cuda.current_stream(dev)      # the capture stream while capturing
        for i, s in enumerate(dev_steps):
            if evs is not None:
                evs[i][0].record(stream)
            if gated:
                gdn.decode_step_gated(s["q"], s["k"], s["v"], s["g"], s["b"], s["A_log"],
                                      s["dt_bias"], w.scale, L2_EPS, st, out=out, stream=stream)
            else:
                gdn.decode_step(s["q"], s["k"], s["v"], s["g"], s["b"], w.scale, st, out=out,
                                stream=stream)
            if evs is not None:
                evs[i][1].record(stream)

    settle(torch, lambda i: run64(), warmup)
    evs = [_events(torch, len(dev_steps)) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        run64(evs[r])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n = reps * len(dev_steps)
    kern_ms = float(np.mean([a.elapsed_time(b) for e in evs for a, b in e]))
    ms_step = (t1 - t0) * 1e3 / n
    # the same passes replayed from a HIP graph captured once (no launch gaps)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run64()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run64()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / n
    return ms_step, kern_ms, decode_algorithmic(w.B, w.Hk, w.Hv, w.Dk, w.Dv), graph_ms


def conv_algorithmic(B, C, T, K, esize=2):
    """HBM bytes of one conv1d call: x read, out written ([B,C,T] each), the
    window state written (prefill) or read and written (decode, T = 1), and
    the fp32 weights [C,K]."""
    state = B * C * K * esize * (2 if T == 1 else 1)
    return float(2 * B * C * T * esize + state + C * K * 4)


def bench_conv(torch, gdn, workloads, name, steps, warmup):
    """Times the conv1d workload ``name`` (prefill: one call per step;
    decode: one token per step, window state carried)."""
    w = workloads.CONV_WORKLOADS[name]
    decode = w.T == 1
    d = workloads.draw_conv(w.B, w.C, w.T, w.K, dtype=w.dtype, decode=decode)
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(d["x"]).to(dev).to(torch.bfloat16)
    wt = torch.from_numpy(d["w"]).to(dev)
    out = torch.empty_like(x)
    if decode:
        st = torch.from_numpy(d["state"]).to(dev).to(torch.bfloat16)
    else:
        st = torch.empty((w.B, w.C, w.K), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i=0):
        if decode:
            gdn.conv1d_decode(x, st, wt, out=out, stream=stream)
        else:
            gdn.conv1d_prefill(x, wt, out=out, state=st, stream=stream)

    settle(torch, step, warmup)
    ev = _events(torch, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    if decode:
        # A decode call lasts a few microseconds, less than the host's launch
        # gap, so events around single launches time the gap. The kernel time
        # comes from CONV_GRAPH_CALLS calls captured once in a HIP graph: the
        # replays run them back to back, one event pair per replay.
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(CONV_GRAPH_CALLS):
                gdn.conv1d_decode(x, st, wt, out=out, stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(CONV_GRAPH_CALLS):
                gdn.conv1d_decode(x, st, wt, out=out,
                                  stream=torch.cuda.current_stream(dev))
        nrep = max(1, steps // CONV_GRAPH_CALLS)
        ev = _events(torch, nrep)
        torch.cuda.synchronize()
        for i in range(nrep):
            ev[i][0].record(stream)
            g.replay()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev])) / CONV_GRAPH_CALLS
    return w, (t1 - t0) * 1e3 / steps, kern_ms, conv_algorithmic(w.B, w.C, w.T, w.K)


CONV_GRAPH_CALLS = 10


def _timed(torch, stream, step, steps, warmup):
    """W untimed calls and the settling calls, then K calls each bracketed by
    events on ``stream``; returns (wall ms per call, mean event ms per call)."""
    settle(torch, step, warmup)
    ev = _events(torch, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_rmsnorm(torch, gdn, steps, warmup):
    """RMSNormGated over the prefill output of the B=4, S=8192 workload."""
    B, Hv, S, Dv = 4, 32, 8192, 128
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(11)
    o = torch.randn((B, Hv, S, Dv), device=dev, generator=g).to(torch.bfloat16)
    z = torch.randn((B, S, Hv, Dv), device=dev, generator=g).to(torch.bfloat16)
    w = 1.0 + 0.1 * torch.randn((Dv,), device=dev, generator=g)
    out = torch.empty_like(z)
    stream = torch.cuda.current_stream(dev)
    ms, kern = _timed(torch, stream, lambda i: gdn.rmsnorm_gated(o, z, w, 1e-6, out=out,
                                                                 stream=stream), steps, warmup)
    nbytes = float(3 * B * Hv * S * Dv * 2 + Dv * 4)
    return dict(B=B, Hv=Hv, S=S, Dv=Dv), ms, kern, nbytes


def bench_decode_block(torch, gdn, workloads, steps, warmup):
    """The fused decode block at B=256, Hk=16, Hv=32, Dk=Dv=128, K=4, bf16:
    eight seeded token draws cycled, conv windows ping-ponged, state carried."""
    B, Hk, Hv, Dk, Dv, K = 256, 16, 32, 128, 128, 4
    dev = torch.device("cuda", 0)
    d0 = workloads.draw_block(B, Hk, Hv, Dk, Dv, K)
    toks = [d0] + [workloads.draw_block(B, Hk, Hv, Dk, Dv, K, step=i, with_state=False)
                   for i in range(1, 8)]
    up = lambda a, bf: torch.from_numpy(a).to(dev).to(torch.bfloat16 if bf else torch.float32)
    dtoks = [{k: up(t[k], k in ("mixed", "z")) for k in ("mixed", "z", "a", "b")} for t in toks]
    fx = {k: up(d0[k], False) for k in ("conv_weight", "A_log", "dt_bias", "norm_weight")}
    st = up(d0["state"], False)
    win = [up(d0["conv_state"], True), up(d0["conv_state"], True)]
    out = torch.empty((B, Hv * Dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = dtoks[i % 8]
        gdn.decode_block(t["mixed"], t["z"], t["a"], t["b"], win[i & 1], fx["conv_weight"],
                         fx["A_log"], fx["dt_bias"], fx["norm_weight"], 1.0 / np.sqrt(Dk), 1e-6,
                         1e-6, st, Hk, Hv, Dk, Dv, conv_state_out=win[(i + 1) & 1], out=out,
                         stream=stream)

    ms, kern = _timed(torch, stream, step, steps, warmup)
    C = 2 * Hk * Dk + Hv * Dv
    nbytes = float(2 * B * Hv * Dk * Dv * 4 + B * C * 2 + B * Hv * Dv * 2 * 2 + B * Hv * 8
                   + 2 * B * C * K * 2 + C * K * 4 + Hv * 8 + Dv * 4)
    return dict(B=B, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K), ms, kern, nbytes


INVERSE_AB_B = 2               # batch of the inverse-method comparison


def bench_inverse_ab(torch, gdn, workloads, w, steps, warmup, lengths=(128, 512, 2048, 8192)):
    """Kernel time of the prefill with each intra-chunk inverse over the first
    S tokens of a draw with the shapes of ``w`` at batch INVERSE_AB_B (state
    carried, as in the main prefill line). The batch differs from the headline
    workload's so that the kernels timed here are other instances than the
    headline's, and a profiler's per-kernel statistics keep the two apart."""
    dev = torch.device("cuda", 0)
    d = workloads.draw_workload(w, B=INVERSE_AB_B)
    rows = []
    for S in lengths:
        t = {k: torch.from_numpy(np.ascontiguousarray(d[k][:, :, :S])).to(dev)
             for k in ("q", "k", "v", "g_log", "beta")}
        for k in ("q", "k", "v"):
            t[k] = t[k].to(torch.bfloat16)
        state = torch.from_numpy(d["state"]).to(dev)
        out = torch.empty((INVERSE_AB_B, w.Hv, S, w.Dv), dtype=torch.bfloat16, device=dev)
        stream = torch.cuda.current_stream(dev)
        row = {"S": S}
        for name, inv in (("substitution", gdn.GDN_INV_SUBSTITUTION),
                          ("neumann", gdn.GDN_INV_NEUMANN)):
            step = lambda i, inv=inv: gdn.chunked_prefill(
                t["q"], t["k"], t["v"], t["g_log"], t["beta"], w.scale, state, out=out,
                stream=stream, inverse=inv)
            _, kern = _timed(torch, stream, step, steps, warmup)
            row[name + "_ms"] = kern
        row["neumann_over_substitution"] = row["neumann_ms"] / row["substitution_ms"]
        rows.append(row)
    return {"B": INVERSE_AB_B, "Hk": w.Hk, "Hv": w.Hv, "Dk": w.Dk, "Dv": w.Dv, "rows": rows,
            "note": "kernel time per call (HIP events); the intra-chunk inverse is blocked "
                    "forward substitution (default) or a Neumann product"}


def bench_copy(torch, mib, steps):
    """Streaming elementwise kernel over ``mib`` MiB of fp32: b = -a reads and
    writes that many bytes once (a same-dtype copy_ would be a DMA transfer,
    which the shader counters do not see)."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    return {"copy_bytes_each_way": n * 4, "ms": dt * 1e3, "GB_s": 2 * n * 4 / dt / 1e9}


def _repeat_for(fn, min_s, max_reps):
    """Calls fn() until at least min_s seconds have passed (at most max_reps
    calls, at least one); returns (calls, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or n >= max_reps:
            return n, dt


def cpu_baseline_prefill(w, d):
    """The oracle on whole steps of the prefill workload (B x S tokens x Hv
    value heads), the state carried from step to step as in the GPU timing,
    repeated for at least 10 s."""
    import oracle
    n = oracle.default_threads()
    st = [d["state"].astype(np.float64)]

    def step():
        _, st[0] = oracle.gdn_serial(d["q"], d["k"], d["v"], d["g_log"], d["beta"], w.scale,
                                     st[0], nthreads=n, inplace=True)
    reps, dt = _repeat_for(step, 10.0, 16)
    return {"value": reps * w.B * w.S / dt, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": "%d whole steps of the prefill workload (%d x %d tokens x %d value heads "
                      "each, state carried), fp64 token-serial, %.1f s" % (reps, w.B, w.S, w.Hv, dt)}


def cpu_baseline_decode(w, steps, state0):
    """The oracle on passes over all decode steps of the workload, state
    carried, repeated for at least 3 s."""
    import oracle
    n = oracle.default_threads()
    st = [state0.astype(np.float64)]

    def run_pass():
        for s in steps:
            _, st[0] = oracle.gdn_serial(s["q"], s["k"], s["v"], s["g_log"], s["beta"], w.scale,
                                         st[0], nthreads=n, inplace=True)
    reps, dt = _repeat_for(run_pass, 3.0, 16)
    return {"value": reps * len(steps) / dt, "unit": "steps/s", "cores": n, "kind": "oracle",
            "sample": "%d pass%s over all %d decode steps at B=%d, state carried, fp64, %.1f s"
                      % (reps, "" if reps == 1 else "es", len(steps), w.B, dt)}


def cpu_baseline_conv(workloads, cw, decode):
    """The conv1d oracle (numpy fp64, one core): prefill on one batch row of
    the workload (all C channels, all T tokens), decode on whole steps, each
    repeated for at least 2 s."""
    from oracle import conv1d
    d = workloads.draw_conv(1 if not decode else cw.B, cw.C, cw.T, cw.K, dtype=cw.dtype,
                         decode=decode)
    if decode:
        reps, dt = _repeat_for(lambda: conv1d.conv1d_decode(d["x"], d["state"], d["w"]), 2.0, 200)
        return {"value": reps / dt, "unit": "steps/s", "cores": 1, "kind": "oracle",
                "sample": "%d decode steps at B=%d, C=%d, K=%d, numpy fp64, %.1f s"
                          % (reps, cw.B, cw.C, cw.K, dt)}
    reps, dt = _repeat_for(lambda: conv1d.conv1d_prefill(d["x"], d["w"]), 2.0, 16)
    return {"value": reps * cw.T / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "one of the %d batch rows (C=%d channels x T=%d tokens, K=%d), run %d "
                      "times, numpy fp64, %.1f s" % (cw.B, cw.C, cw.T, cw.K, reps, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "prefill_gated", "decode_gated",
                                       "conv_prefill", "conv_decode", "rmsnorm", "decode_block",
                                       "inverse_ab", "copy"], default=None)
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the recurrence has no cross-GPU step in this "
              "library (per-GPU shards of (batch, key-head group) are independent); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_chunked_amd as gdn
    import workloads
    gdn.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.only == "copy":
        print(json.dumps({"copy": bench_copy(torch, args.copy_mib, args.steps)}), flush=True)
        return
    reps, dwarm = max(1, args.steps // 10), max(1, args.warmup // 10)
    dw = workloads.WORKLOADS["decode_b256"]
    w = workloads.WORKLOADS["prefill_b4_s8192"]
    if args.only in ("decode", "decode_gated"):
        dstate0, dsteps = workloads.draw_decode_steps(dw, raw=True)
        dms, dkern_ms, dbytes, _ = bench_decode(torch, gdn, dw, dstate0, dsteps, reps, dwarm,
                                                gated=args.only == "decode_gated")
        print(json.dumps({args.only + "_ms_per_step": dms, "kernel_ms": dkern_ms,
                          "GB_s": dbytes / (dkern_ms / 1e3) / 1e9}), flush=True)
        return
    if args.only == "inverse_ab":
        print(json.dumps({"inverse_ab": bench_inverse_ab(torch, gdn, workloads, w, args.steps,
                                                         args.warmup)}), flush=True)
        return
    if args.only == "rmsnorm":
        _, ms, kern, nb = bench_rmsnorm(torch, gdn, args.steps, args.warmup)
        print(json.dumps({"rmsnorm_ms": ms, "kernel_ms": kern, "GB_s": nb / (kern / 1e3) / 1e9}),
              flush=True)
        return
    if args.only == "decode_block":
        _, ms, kern, nb = bench_decode_block(torch, gdn, workloads, args.steps, args.warmup)
        print(json.dumps({"decode_block_ms": ms, "kernel_ms": kern,
                          "GB_s": nb / (kern / 1e3) / 1e9}), flush=True)
        return
    if args.only in ("conv_prefill", "conv_decode"):
        name = {"conv_prefill": "conv_prefill_b4_t8192", "conv_decode": "conv_decode_b256"}
        cw, cms, ckern_ms, cbytes = bench_conv(torch, gdn, workloads, name[args.only], args.steps,
                                               args.warmup)
        print(json.dumps({args.only + "_ms_per_step": cms, "kernel_ms": ckern_ms,
                          "GB_s": cbytes / (ckern_ms / 1e3) / 1e9}), flush=True)
        return
    if args.only in ("prefill", "prefill_gated"):
        d = workloads.draw_workload(w, raw=True)
        ms_step, kern_ms, _, _ = bench_prefill(torch, gdn, w, d, args.steps, args.warmup,
                                               gated=args.only == "prefill_gated")
        print(json.dumps({args.only + "_ms_per_step": ms_step, "kernel_ms": kern_ms,
                          "tokens_per_s": w.B * w.S / (ms_step / 1e3)}), flush=True)
        return
    # Decode first, then prefill: the GPU needs ~100 ms under load to reach its
    # steady clocks, and the decode passes (with their own warm-up) supply it
    # before the prefill's warm-up steps.
    dstate0, dsteps = workloads.draw_decode_steps(dw, raw=True)
    dms, dkern_ms, dbytes, dgraph_ms = bench_decode(torch, gdn, dw, dstate0, dsteps, reps, dwarm)
    progress("decode %.4f ms/step" % dms)
    gdms, gdkern_ms, _, gdgraph_ms = bench_decode(torch, gdn, dw, dstate0, dsteps, reps, dwarm,
                                                  gated=True)
    d = workloads.draw_workload(w, raw=True)
    clocks = []
    ms_step, kern_ms, nbytes, flops = bench_prefill(torch, gdn, w, d, args.steps, args.warmup,
                                                    clocks=clocks)
    progress("prefill %.4f ms/step (kernel %.4f ms)" % (ms_step, kern_ms))
    gms_step, gkern_ms, _, _ = bench_prefill(torch, gdn, w, d, args.steps, args.warmup,
                                             gated=True)
    progress("prefill gated %.4f ms/step" % gms_step)
    # The single-sequence workloads (B = 1): S = 2048 from a zero state, and
    # S = 65536 from a carried state with standard and strong decay.
    long_rows = {}
    for wname, variant in (("prefill_s2048", "std"), ("prefill_s65536", "std"),
                           ("prefill_s65536", "strong")):
        wl = workloads.WORKLOADS[wname]
        dl = workloads.draw_workload(wl, variant=variant)
        lms, lkern, lbytes, lflops = bench_prefill(torch, gdn, wl, dl, args.steps, args.warmup)
        del dl
        long_rows[(wname, variant)] = (wl, lms, lkern, lbytes, lflops)
        progress("%s %s %.4f ms/step" % (wname, variant, lms))
    cpw, cpms, cpkern, cpbytes = bench_conv(torch, gdn, workloads, "conv_prefill_b4_t8192",
                                            args.steps, args.warmup)
    cdw, cdms, cdkern, cdbytes = bench_conv(torch, gdn, workloads, "conv_decode_b256",
                                            10 * args.steps, args.warmup)
    rcfg, rms_ms, rms_kern, rms_bytes = bench_rmsnorm(torch, gdn, args.steps, args.warmup)
    bcfg, blk_ms, blk_kern, blk_bytes = bench_decode_block(torch, gdn, workloads, args.steps,
                                                           args.warmup)
    tokens = w.B * w.S
    hbm = lambda b, ms: {"achieved": b / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "kernel_ms": ms,
                         "algorithmic_bytes_per_launch": b}
    res = {
        "metric": METRIC,
        "value": tokens / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; normalised q/k, gates from random A_log/dt_bias)",
        "config": {"workload": "prefill_b4_s8192", "B": w.B, "Hk": w.Hk, "Hv": w.Hv,
                   "S": w.S, "Dk": w.Dk, "Dv": w.Dv, "tokens_per_step": tokens,
                   "state": "fp32 in place, carried across steps"},
        "roofline": dict(bound="hbm", kernel="gdn_prefill_kernel",
                         traffic=measured_traffic("gdn_prefill_kernel"), **hbm(nbytes, kern_ms)),
        "mfma_util": mfma_util(flops, kern_ms, w, mfma_counters("gdn_prefill_kernel", kern_ms)),
        "sclk": clock_record(clocks),
        "decode": {"workload": "decode_b256", "B": dw.B, "Hk": dw.Hk, "Hv": dw.Hv,
                   "value": 1e3 / dms, "unit": "steps/s", "ms_per_step": dms,
                   "tokens_per_s": dw.B * 1e3 / dms,
                   "graph": {"value": 1e3 / dgraph_ms, "ms_per_step": dgraph_ms,
                             "note": "the 64-step pass captured once in a HIP graph and replayed"},
                   "roofline": dict(bound="hbm", kernel="gdn_decode_kernel",
                                    traffic=measured_traffic("gdn_decode_kernel"),
                                    **hbm(dbytes, dkern_ms))},
        "prefill_gated": {"workload": "prefill_b4_s8192 (raw q/k, a, b, A_log, dt_bias)",
                          "value": tokens / (gms_step / 1e3), "unit": "tokens/s",
                          "ms_per_step": gms_step, "l2_eps": L2_EPS,
                          "roofline": dict(bound="hbm", kernel="gdn_prefill_kernel (gated)",
                                           traffic=measured_traffic("gdn_prefill_kernel_gated"),
                                           **hbm(nbytes, gkern_ms))},
        "decode_gated": {"workload": "decode_b256 (raw q/k, a, b, A_log, dt_bias)",
                         "value": 1e3 / gdms, "unit": "steps/s", "ms_per_step": gdms,
                         "graph": {"value": 1e3 / gdgraph_ms, "ms_per_step": gdgraph_ms},
                         "l2_eps": L2_EPS,
                         "roofline": dict(bound="hbm", kernel="gdn_decode_kernel (gated)",
                                          traffic=measured_traffic("gdn_decode_kernel_gated"),
                                          **hbm(dbytes, gdkern_ms))},
        "prefill_s2048": long_section(long_rows[("prefill_s2048", "std")], hbm),
        "prefill_s65536": {v: long_section(long_rows[("prefill_s65536", v)], hbm)
                           for v in ("std", "strong")},
        "conv1d_prefill": {"workload": cpw.name, "B": cpw.B, "C": cpw.C, "T": cpw.T,
                           "K": cpw.K, "value": cpw.B * cpw.T / (cpms / 1e3),
                           "unit": "tokens/s", "ms_per_step": cpms,
                           "roofline": dict(bound="hbm", kernel="gdn_conv1d_prefill_tile_kernel",
                                            traffic=measured_traffic("gdn_conv1d_prefill_tile_kernel"),
                                            **hbm(cpbytes, cpkern))},
        "conv1d_decode": {"workload": cdw.name, "B": cdw.B, "C": cdw.C, "K": cdw.K,
                          "value": 1e3 / cdms, "unit": "steps/s", "ms_per_step": cdms,
                          "roofline": dict(bound="hbm", kernel="gdn_conv1d_decode_kernel",
                                           traffic=measured_traffic("gdn_conv1d_decode_kernel"),
                                           **hbm(cdbytes, cdkern))},
        "rmsnorm_gated": dict(workload="prefill_b4_s8192 output", value=rcfg["B"] * rcfg["S"]
                              / (rms_ms / 1e3), unit="tokens/s", ms_per_step=rms_ms,
                              roofline=dict(bound="hbm", kernel="gdn_rmsnorm_gated_kernel",
                                            traffic=measured_traffic("gdn_rmsnorm_gated_kernel"),
                                            **hbm(rms_bytes, rms_kern)), **rcfg),
        "decode_block": dict(workload="decode_block_b256", value=1e3 / blk_ms, unit="steps/s",
                             ms_per_step=blk_ms,
                             roofline=dict(bound="hbm", kernel="gdn_decode_kernel (block)",
                                           traffic=measured_traffic("gdn_decode_kernel_block"),
                                           **hbm(blk_bytes, blk_kern)), **bcfg),
        "host": {"cpu": platform.processor() or platform.machine(),
                 "gpu": torch.cuda.get_device_name(0)},
    }
    # The inverse-method comparison runs last, at another batch (other kernel
    # instances than the headline's).
    res["inverse_ab"] = bench_inverse_ab(torch, gdn, workloads, w, max(5, args.steps // 2),
                                         args.warmup)
    progress("inverse A/B done")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w, d)
        res["decode"]["cpu_baseline"] = cpu_baseline_decode(dw, dsteps, dstate0)
        res["conv1d_prefill"]["cpu_baseline"] = cpu_baseline_conv(workloads, cpw, False)
        res["conv1d_decode"]["cpu_baseline"] = cpu_baseline_conv(workloads, cdw, True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Host-side checks of bench.py: the one-GPU guard, the algorithmic byte and
flop counts that its roofline figures divide by (worked out here term by
term for the bench workloads), and the source digest that keys the committed
counter summaries to the kernel code."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_algorithmic_bench_workload():
    """B=4, Hk=16, Hv=32, S=8192, Dk=Dv=128, bf16 q/k/v/out, fp32 g, beta and state."""
    tokens = 4 * 8192
    qk = 2 * 16 * 128 * 2            # q and k rows of one token, all key heads
    vo = 2 * 32 * 128 * 2            # v and out rows, all value heads
    gb = 32 * 2 * 4                  # g and beta
    state = 2 * (4 * 32 * 128 * 128 * 4)   # read once and written once
    assert qk + vo + gb == 24832
    nbytes, flops = bench.prefill_algorithmic(4, 16, 32, 8192, 128, 128)
    assert nbytes == tokens * (qk + vo + gb) + state == 830_472_192
    # flops of one chunk of C tokens: per value head T K and T V (triangle:
    # half of 2 C^2 D each), K S0 / Q S0 / K^T U (2 C Dk Dv each), P U (half
    # of 2 C^2 Dv), the inverse (C^3 / 3); per key head K K^T and Q K^T (half
    # of 2 C^2 Dk each). The reported count uses C = 64: 4.24 MFLOP per token.
    for C, total in ((64, 138_870_609_237.33), (32, 120_616_998_229.33)):
        per_vh = C * C * 128 * 2 + 3 * 2 * C * 128 * 128 + C * C * 128 + C ** 3 / 3
        per_kh = 2 * C * C * 128
        chunks = tokens // C
        f = bench.prefill_algorithmic(4, 16, 32, 8192, 128, 128, chunk=C)[1]
        assert abs(f - chunks * (32 * per_vh + 16 * per_kh)) < 1.0
        assert abs(f - total) < 1.0, (C, f)
    assert abs(flops - 138_870_609_237.33) < 1.0          # the default count: C = 64
    assert 4.23e6 < flops / tokens < 4.24e6


def test_mfma_util_reports_fixed_count(monkeypatch):
    """frac = 64-token count / kernel time / 2.5 PFLOP/s; the 32-token count beside it."""
    import workloads
    w = workloads.WORKLOADS["prefill_b4_s8192"]
    nbytes, flops = bench.prefill_algorithmic(w.B, w.Hk, w.Hv, w.S, w.Dk, w.Dv)
    u = bench.mfma_util(flops, 0.5, w)
    assert abs(u["frac"] - flops / 0.5e-3 / 2.5e15) < 1e-12
    assert abs(u["kernel_chunk32"]["frac"] - 120_616_998_229.33 / 0.5e-3 / 2.5e15) < 1e-9
    assert abs(u["flops_per_token"] - flops / (4 * 8192)) < 1e-6


def test_settle_runs_warmup_then_busy_time():
    """The settling phase runs at least the W warm-up calls and then keeps
    the device busy for the minimum time (here with a fake torch)."""
    import time

    class FakeCuda:
        @staticmethod
        def synchronize():
            pass

    class FakeTorch:
        cuda = FakeCuda

    calls = []
    t0 = time.perf_counter()
    n = bench.settle(FakeTorch, lambda i: calls.append(i), 3, min_ms=20.0)
    assert (time.perf_counter() - t0) * 1e3 >= 20.0
    assert n == len(calls) >= 3 + 8


def test_decode_and_conv_algorithmic_bench_workloads():
    # decode at B=256: the fp32 state read and written dominates
    state = 2 * (256 * 32 * 128 * 128 * 4)
    vectors = 2 * 256 * 16 * 128 * 2 + 2 * 256 * 32 * 128 * 2 + 256 * 32 * 8
    assert bench.decode_algorithmic(256, 16, 32, 128, 128) == state + vectors == 1_080_098_816
    # conv1d prefill: x read and out written, window state written, fp32 taps
    assert bench.conv_algorithmic(4, 8192, 8192, 4) == (
        2 * 4 * 8192 * 8192 * 2 + 4 * 8192 * 4 * 2 + 8192 * 4 * 4) == 1_074_135_040
    # conv1d decode (T = 1): the window state is read and written
    assert bench.conv_algorithmic(256, 8192, 1, 4) == 2 * 256 * 8192 * 2 + 2 * 256 * 8192 * 4 * 2 + 8192 * 4 * 4


def test_source_digest_ignores_comments_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setitem(bench.KERNEL_SOURCES, "k", str(src))
    src.write_text("// header\nint f(int a) { return a + 1; } /* note */\n")
    d1 = bench.source_digest("k")
    src.write_text("/* another\n   header */\nint f(int a) {\n    return a + 1;   // same code\n}\n")
    assert bench.source_digest("k") == d1
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.source_digest("k") != d1

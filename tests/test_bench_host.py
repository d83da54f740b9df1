"""Host-side logic of bench.py: byte model, link-byte report, traffic lookup and
the single-GPU guard. No GPU and no library calls."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_model_bytes_llama3_70b_prefill():
    # R=4, T=8192, H=8192, INT4, g=128 (g2=128), 2-byte activations
    mb = bench.model_bytes(4, 8192, 8192, 4, 128, 128)
    n = 4 * 8192 * 8192
    k1 = n * 2 + n // 2 + n // 128 * 4
    pay2 = 8192 * 8192 // 2 + 8192 * 8192 // 128 * 4
    assert mb["k1"] == k1 == 679477248
    assert mb["k2"] == (k1 - n * 2) + pay2 == 178257920
    assert mb["k3"] == pay2 + 8192 * 8192 * 2 == 169869312
    assert mb["total"] == mb["k1"] + mb["k2"] + mb["k3"]


def test_model_bytes_wide_group_uses_stage2_group():
    # g=4096 > C=1024: stage-1 metadata per 4096 columns, stage-2 per 1024
    mb = bench.model_bytes(4, 16, 4096, 8, 4096, 1024)
    n = 4 * 16 * 4096
    assert mb["k1"] == n * 2 + n + n // 4096 * 4
    assert mb["k3"] == 16 * 4096 + 16 * 4096 // 1024 * 4 + 16 * 4096 * 2


def test_link_bytes_ratio_int4_g128():
    # 16-bit ring vs two-step codec: 16 / (4 + 32/128) = 3.7647
    lb = bench.link_bytes(4, 8192, 8192, 4, 128, 128)
    assert abs(lb["ratio"] - 16 / (4 + 32 / 128)) < 1e-3


def test_traffic_only_for_the_profiled_workload():
    # The committed counter summary covers one workload and one K1 source.
    other = bench.measured_traffic("decode")
    assert other is None
    v = bench.measured_traffic("llama3_70b_prefill")
    if v is not None:    # present only while the K1 source is the profiled one
        mb = bench.model_bytes(4, 8192, 8192, 4, 128, 128)
        assert 0.95 < v / mb["k1"] < 1.2


def test_more_than_one_gpu_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "single GPU" in msg["error"]


class _FakeEvent:
    """Stands in for torch.cuda.Event: elapsed_time() replays scripted block times."""
    script = []

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self, stream=None):
        pass

    def elapsed_time(self, other):
        return _FakeEvent.script.pop(0)


class _FakeTorch:
    class cuda:
        Event = _FakeEvent

        @staticmethod
        def synchronize():
            pass


def test_settle_waits_for_min_time_and_two_agreeing_blocks():
    # probe: 3 calls in 3 ms -> 1 ms per call -> blocks of SETTLE_BLOCK_MS calls
    blk = bench.SETTLE_BLOCK_MS
    n = int(round(blk))
    per_call = [1.30, 1.25, 1.10, 1.02, 1.001, 1.0, 1.0, 1.0] + [1.0] * 200
    _FakeEvent.script = [3.0] + [p * n for p in per_call]
    calls = []
    st = bench.settle_clock(_FakeTorch, lambda: calls.append(1), None, min_ms=30.0, max_ms=500.0)
    assert st["steady"]
    # stops at the first block with >= 30 ms behind it whose time is within 1% of the last
    elapsed, k = 0.0, 0
    while True:
        elapsed += per_call[k] * n
        if elapsed >= 30.0 and k >= 1 and abs(per_call[k] - per_call[k - 1]) <= 0.01 * per_call[k - 1]:
            break
        k += 1
    assert st["ms"] == round(elapsed, 2)
    assert st["calls"] == 6 + (k + 1) * n == len(calls)
    assert st["first_block_ms_per_call"] == round(per_call[0], 5)


def test_settle_gives_up_at_max_time():
    _FakeEvent.script = [3.0] + [float(i % 2 + 1) * 6 for i in range(1000)]
    st = bench.settle_clock(_FakeTorch, lambda: None, None, min_ms=10.0, max_ms=100.0)
    assert not st["steady"] and st["ms"] >= 100.0


def test_host_info_names_the_processor_count():
    hi = bench.host_info()
    assert hi["host_nproc"] == os.cpu_count()
    assert "platform" in hi


def test_k1_hash_ignores_comments_but_not_code():
    src = "int a = 1; // one\n/* block\n comment */ int b = a + 2;\n"
    assert bench.code_only(src) == "int a = 1; int b = a + 2;"
    assert bench.code_only(src.replace("// one", "// a different note")) == bench.code_only(src)
    assert bench.code_only(src.replace("a + 2", "a + 3")) != bench.code_only(src)


def test_k1_counter_summary_is_for_the_current_code():
    """The committed HBM-counter summary was measured on K1's current code (so
    bench.py reports roofline.traffic); a change to K1's code needs a new
    counter run."""
    assert bench.measured_traffic("llama3_70b_prefill") is not None


def test_k2_counter_summary_is_for_the_current_code():
    """The committed counter summary of K2 (VALU instructions per launch, for its ALU
    roofline) was measured on K2's current code."""
    v = bench.measured_k2_valu("llama3_70b_prefill")
    assert v is not None
    # 16.2 VALU instructions per output position, 8192 x 8192 positions, 64 lanes
    assert abs(v * 64 / (8192 * 8192) - 16.19) < 0.05
    assert bench.measured_k2_valu("decode") is None


def test_alu_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs, a wave64 instruction every 4 cycles, 2.4 GHz
    assert abs(bench.PEAK_VALU_G_WAVE_INSTR - 614.4) < 1e-9

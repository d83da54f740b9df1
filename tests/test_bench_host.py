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


def test_k1_event_sampling_stride():
    """K1 is bracketed by events on every 10th timed step, keeping at least 20
    samples when the run allows it, and every step of a short run."""
    assert bench.k1_sample_every(200) == 10
    assert bench.k1_sample_every(1000) == 10
    assert bench.k1_sample_every(100) == 5
    assert bench.k1_sample_every(20) == 1
    assert bench.k1_sample_every(5) == 1
    for k in (1, 7, 40, 199, 200, 5000):
        every = bench.k1_sample_every(k)
        assert len(range(0, k, every)) >= min(k, 20)


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

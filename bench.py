"""Benchmark of the low-bit all-reduce codec on one MI355X.

One step = one pass of the whole path over one batch of synthetic operands:
quantize the R operands (K1), dequantize-sum-requantize every hidden chunk
(K2), dequantize the gathered result (K3) -- the quantize / Reduce-Scatter /
requantize / All-Gather / dequantize sequence of "Flash Communication:
Reducing Tensor Parallelization Bottleneck for Fast Large Language Model
Inference" (Figure 5, right), with the two exchanges as HBM hand-offs.

Workload: the LLaMA-3-70B prefill all-reduce of Figure 1 (batch 8 x 1024
tokens, TP = 4): R=4 operands of T=8192 x H=8192 bf16, 4-bit codes, groups
of 128. Inputs are seeded synthetic activations, resident in HBM before the
timed region.

Metric: algorithmic HBM bytes per step / time per step (GB/s). Algorithmic
bytes: every input read once, each payload written once and read once, the
output written once (scales and zeros 4 bytes per group).

Order of a run:
  1. settle: pipeline steps back to back until the time per step is steady
     (after idle, the GPU's power management holds the engine clock down for
     the first ~15 ms of load; the path's steady state is what is measured);
  2. W warm-up steps, then exactly K timed steps with no event in the stream
     (the timed region is bracketed by device synchronizations only);
  3. a separate pass of 50 steps with HIP events around each kernel, on the
     same stream: per-kernel times and K1's roofline (K1 moves two thirds of
     the bytes);
  4. the same K steps after an idle second (the cold-start figure);
  5. the streaming ceilings (always), then the other workloads (LLaMA-3-8B
     prefill, the group-size sweep with its errors, a group length that is not
     a power of two, decode and tiny latency back to back, in a HIP graph and
     from cold caches), the uncompressed comparator, the residual-add and
     linear-layer fusions, the CPU oracle.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for quant->dequant-sum-requant->dequant"
WORKLOAD = "llama3_70b_prefill"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16/fp16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_llama3_70b_prefill_traffic.txt")
K1_SOURCES = ("bit_activation_compression_amd/csrc/fc_quantize.hip",
              "bit_activation_compression_amd/csrc/fc_device.h")
K2_COUNTER_FILE = os.path.join(ROOT, "profiles", "dsr_llama3_70b_prefill_counters.md")
K2_SOURCES = ("bit_activation_compression_amd/csrc/fc_dequant_sum_requant.hip",
              "bit_activation_compression_amd/csrc/fc_device.h")
# VALU issue peak of the chip: 256 compute units x 4 SIMDs, one wave64 instruction per
# SIMD every 4 cycles (16 lanes wide), at 2.4 GHz (non-packed instructions)
PEAK_VALU_G_WAVE_INSTR = 256 * 4 * 2.4 / 4

BREAKDOWN_STEPS = 50   # steps of the per-kernel event pass
GRAPH_CALLS = 20       # calls captured per HIP graph in the launch-bound measurements
LINEAR_ROUNDS = 3      # interleaved timing rounds of the linear-layer variants
SWEEP_SETS = 4         # operand copies of the sweep (134 MB each) read in turn
GENERIC_SETS = 3       # and of the generic-group shape (168 MB each)
EVICT_BYTES = 1 << 30  # scratch written before each cache-cold call (L2s and the 256 MB Infinity Cache)
COLD_CALLS = 30        # cache-cold calls timed one by one
CPU_PASSES = 3         # passes of the CPU oracle over the whole workload (~4-5 s each)
SETTLE_MIN_MS = 60.0   # least back-to-back time before the clock is taken as steady
SETTLE_MAX_MS = 800.0
SETTLE_BLOCK_MS = 6.0
COLD_IDLE_S = 1.0


def model_bytes(R: int, T: int, H: int, bits: int, group: int, group2: int, e: int = 2,
                bits2: int | None = None) -> dict:
    bits2 = bits if bits2 is None else bits2
    n1, n2 = R * T * H, T * H
    p1 = n1 * bits // 8 + n1 // group * 4
    p2 = n2 * bits2 // 8 + n2 // group2 * 4
    k1 = n1 * e + p1
    k2 = p1 + p2
    k3 = p2 + n2 * e
    return {"k1": k1, "k2": k2, "k3": k3, "total": k1 + k2 + k3, "payload1": p1, "payload2": p2}


def link_bytes(R: int, T: int, H: int, bits: int, group: int, group2: int, e: int = 2) -> dict:
    """Bytes one rank would send over the links for one all-reduce of a [T][H] tensor: a ring
    all-reduce of 16-bit values (2(R-1) hops of 1/R of the tensor) vs the two-step codec
    (reduce-scatter of its payload-1 chunks, all-gather of its payload-2 chunk)."""
    ring = 2 * (R - 1) * T * H * e // R
    rs = (R - 1) * (T * (H // R) * bits // 8 + T * (H // R) // min(group, H // R) * 4) if group <= H // R \
        else (R - 1) * (T * (H // R) * bits // 8 + T * (H // group) * 4)
    ag = (R - 1) * (T * (H // R) * bits // 8 + T * (H // R) // group2 * 4)
    return {"ring_16bit": ring, "two_step_codec": rs + ag, "ratio": round(ring / (rs + ag), 3)}


def code_only(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed: what a
    comment edit leaves unchanged. (The kernel sources hold no string literals
    that contain comment markers.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(sources=K1_SOURCES) -> str:
    """Hash of a kernel's code (comments and layout ignored): a counter summary is
    valid while the code it was measured on is unchanged."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def k1_source_hash() -> str:
    return source_hash(K1_SOURCES)


def measured_k2_valu(workload: str) -> float | None:
    """VALU wave-instructions per K2 launch (SQ_INSTS_VALU) from the committed counter
    summary, if it was taken on this workload and on the current K2 source."""
    if not os.path.exists(K2_COUNTER_FILE):
        return None
    txt = open(K2_COUNTER_FILE).read()
    m_w = re.search(r"^workload:\s*(\S+)", txt, re.M)
    m_src = re.search(r"^k2_source_sha256_16:\s*(\S+)", txt, re.M)
    m_v = re.search(r"^k2_valu_wave_instructions_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_w or m_w.group(1) != workload or not m_src or not m_v:
        return None
    if m_src.group(1) != source_hash(K2_SOURCES):
        return None
    return float(m_v.group(1))


def measured_traffic(workload: str) -> float | None:
    """L2-to-fabric bytes per K1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), if it was taken on this
    workload and on the current K1 source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_w = re.search(r"^workload:\s*(\S+)", txt, re.M)
    m_src = re.search(r"^k1_source_sha256_16:\s*(\S+)", txt, re.M)
    m_b = re.search(r"^k1_hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_w or m_w.group(1) != workload:
        return None
    if not m_src or not m_b or m_src.group(1) != k1_source_hash():
        return None
    return float(m_b.group(1))


def host_info() -> dict:
    """The host the CPU oracle ran on: /proc/cpuinfo fields, logical CPUs in the machine
    and in this process's affinity set."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break
                    continue
                k, v = (p.strip() for p in line.split(":", 1))
                if k in ("vendor_id", "model name", "cpu family", "model", "stepping", "cpu MHz",
                         "cache size") and k not in info:
                    info[k] = v
    except OSError:
        pass
    info["host_nproc"] = os.cpu_count()
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    info["platform"] = platform.platform()
    return info


def kernel_rooflines(mb: dict, k_avg, workload: str) -> dict:
    """K2 against the VALU issue peak (it is bound by vector-ALU issue, not HBM) and K3
    against the HBM peak, with the per-kernel event times of the breakdown pass."""
    valu = measured_k2_valu(workload)
    k2_s, k3_s = float(k_avg[1]) * 1e-3, float(k_avg[2]) * 1e-3
    k2 = {"bound": "alu", "unit": "G VALU wave-instructions/s", "peak": PEAK_VALU_G_WAVE_INSTR,
          "achieved": None, "frac": None, "valu_wave_instructions_per_launch": valu,
          "hbm_gbps": round(mb["k2"] / k2_s / 1e9, 1),
          "hbm_frac": round(mb["k2"] / k2_s / 1e9 / PEAK_HBM_GBPS, 4),
          "note": "instructions: SQ_INSTS_VALU from the committed counter summary (null when it "
                  "was measured on other K2 code); peak: 256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles per "
                  "wave64 instruction"}
    if valu is not None:
        a = valu / k2_s / 1e9
        k2.update({"achieved": round(a, 1), "frac": round(a / PEAK_VALU_G_WAVE_INSTR, 4)})
    a3 = mb["k3"] / k3_s / 1e9
    k3 = {"bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBPS, "achieved": round(a3, 1),
          "frac": round(a3 / PEAK_HBM_GBPS, 4)}
    return {"k2_dequant_sum_requant": k2, "k3_dequantize": k3,
            "timing": "HIP events of the 50-step per-kernel pass (dispatch gap included)"}


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def settle_clock(torch, fn, stream, min_ms=SETTLE_MIN_MS, max_ms=SETTLE_MAX_MS) -> dict:
    """Run fn() back to back until the time per call is steady: blocks of ~SETTLE_BLOCK_MS,
    each bracketed by events (between blocks only), until at least min_ms have passed and two
    consecutive blocks agree within 1% (or max_ms is reached)."""
    for _ in range(3):
        fn()
    e = _events(torch, 2)
    e[0].record(stream)
    for _ in range(3):
        fn()
    e[1].record(stream)
    torch.cuda.synchronize()
    per = max(e[0].elapsed_time(e[1]) / 3, 1e-3)
    block = max(1, int(round(SETTLE_BLOCK_MS / per)))
    times, total, calls = [], 0.0, 6
    while True:
        e = _events(torch, 2)
        e[0].record(stream)
        for _ in range(block):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        ms = e[0].elapsed_time(e[1])
        total += ms
        calls += block
        times.append(ms / block)
        if total >= min_ms and len(times) >= 2 and abs(times[-1] - times[-2]) <= 0.01 * times[-2]:
            steady = True
            break
        if total >= max_ms:
            steady = False
            break
    return {"calls": calls, "ms": round(total, 2), "steady": steady,
            "first_block_ms_per_call": round(times[0], 5), "last_block_ms_per_call": round(times[-1], 5)}


def timed_calls(torch, fn, stream, n) -> float:
    """ms per call of n back-to-back calls, events around the whole run."""
    e = _events(torch, 2)
    e[0].record(stream)
    for _ in range(n):
        fn()
    e[1].record(stream)
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) / n


def cold_us_per_call(torch, fn, stream, scratch, n: int = COLD_CALLS) -> float:
    """Median microseconds of n calls, each timed on its own with HIP events right after a
    1 GiB scratch write on the same stream (outside the events), so that neither the L2s nor
    the Infinity Cache hold the call's inputs or payloads."""
    ev = _events(torch, 2 * n)
    for i in range(n):
        scratch.fill_(i & 0xFF)
        ev[2 * i].record(stream)
        fn()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    us = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(n))
    return us[n // 2]


def stage_errors(torch, fc, xf, out, ws, R, T, H, bits, bits2, g, g2) -> dict:
    """Per-element MSE of each stage, from the payloads the library wrote (torch on the GPU):
      stage1_mse: mean over r, t, h of (dequantized payload 1 - x)^2
      stage2_mse: mean of (dequantized payload 2 - sum_r dequantized payload 1)^2
      total_mse : mean of (output - sum_r x)^2, the sum in binary32."""
    v = fc.workspace_views(ws, R, T, H, bits, g, bits2=bits2)
    s1 = v["s1"].view(torch.float16).float().repeat_interleave(g, dim=2)
    z1 = v["z1"].view(torch.float16).float().repeat_interleave(g, dim=2)
    c1 = v["codes1"]
    q1 = torch.stack([c1 & 15, c1 >> 4], dim=-1).reshape(R, T, H) if bits == 4 else c1
    xh32 = q1.float() * s1 + z1
    y = xh32[0].clone()
    for r in range(1, R):
        y = y + xh32[r]
    s2 = v["s2"].view(torch.float16).float().repeat_interleave(g2, dim=1)
    z2 = v["z2"].view(torch.float16).float().repeat_interleave(g2, dim=1)
    c2 = v["codes2"]
    q2 = torch.stack([c2 & 15, c2 >> 4], dim=-1).reshape(T, H) if bits2 == 4 else c2
    yh = q2.float() * s2 + z2
    exact = xf.sum(dim=0)
    return {"stage1_mse": float(((xh32 - xf) ** 2).mean()),
            "stage2_mse": float(((yh - y) ** 2).mean()),
            "total_mse": float(((out.float() - exact) ** 2).mean()),
            "exact_sum_power": float((exact ** 2).mean())}


def quality_report(seed: int) -> int:
    """Error of the codec at each stage, as in Figure 4 (activation quantization with blocks
    from the hidden length down to 128) and Figure 5 right (quantization before the
    Reduce-Scatter vs before the All-Gather), on the synthetic operands; plus throughput.
    The codec runs in the library's kernels; the error statistics (and the binary32
    dequantized values they need) are computed with torch on the GPU from the payloads
    the library wrote. Prints one JSON line with a record per configuration."""
    import numpy as np
    import torch

    import bit_activation_compression_amd as fc
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    names = [f"sweep_int{b}_g{g}" for b in synth.SWEEP_BITS for g in synth.SWEEP_GROUPS]
    names += ["tiny", "llama3_8b_prefill", "llama3_70b_prefill", "decode"]
    widths = {n: [(synth.workload(n).bits, synth.workload(n).bits)] for n in names}
    widths["llama3_70b_prefill"] += [(4, 8), (8, 4), (8, 8)]
    widths["llama3_8b_prefill"] += [(4, 8), (8, 4), (8, 8)]
    records = []
    for name in names:
        w = synth.workload(name)
        R, T, H, g = w.R, w.T, w.H, w.group
        tdt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float16
        x_host = synth.operands(w, seed)
        xd = torch.from_numpy(x_host.view(np.int16)).to(dev).view(tdt)
        xf = xd.float()
        for bits, bits2 in widths[name]:
            g2 = fc.fc_stage2_group(R, H, g)
            out, ws = fc.fc_allreduce_emulated(xd, bits, g, bits2=bits2)
            rec = {"workload": name, "bits_rs": bits, "bits_ag": bits2, "group": g, "group2": g2}
            rec.update(stage_errors(torch, fc, xf, out, ws, R, T, H, bits, bits2, g, g2))

            def call():
                fc.fc_allreduce_emulated(xd, bits, g, out, ws, stream=stream, bits2=bits2)

            settle_clock(torch, call, stream, min_ms=30.0)
            ms = timed_calls(torch, call, stream, 20)
            total = model_bytes(R, T, H, bits, g, g2, bits2=bits2)["total"]
            rec.update({"us_per_call": round(ms * 1e3, 2), "gbps": round(total / (ms * 1e-3) / 1e9, 1)})
            records.append(rec)
            print(f"[quality] {name} int{bits}->int{bits2}: stage1 {rec['stage1_mse']:.4g} "
                  f"stage2 {rec['stage2_mse']:.4g} total {rec['total_mse']:.4g} "
                  f"{rec['us_per_call']} us {rec['gbps']} GB/s", file=sys.stderr, flush=True)
        del xd, xf
    print(json.dumps({"quality": records, "seed": seed, "data": "synthetic",
                      "timing": "us_per_call: 20 back-to-back calls through the Python binding "
                                "(with bits2 given, the mixed-width entry point) after a settle "
                                "run; decode-sized calls are then bound by the host's launch "
                                "cost (the benchmark's decode leg reports graph and cache-cold "
                                "figures)"}))
    return 0


def graph_us_per_call(torch, call, stream, dev) -> float:
    """GRAPH_CALLS consecutive calls captured in one HIP graph (as a serving step would be)
    and replayed; microseconds per call."""
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        call(cap)
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(GRAPH_CALLS):
                call(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    settle_clock(torch, graph.replay, stream, min_ms=30.0)
    ms = timed_calls(torch, graph.replay, stream, 20)
    del graph
    return ms * 1e3 / GRAPH_CALLS


def other_workloads(torch, np, fc, synth, seed, dev, stream) -> dict:
    """The other configurations of the path on the same clock: LLaMA-3-8B prefill and the
    group-size sweep (GB/s, and the sweep's per-stage errors, Figure 4's trend), decode
    (microseconds per call: one eager launch, inside a HIP graph, and the three stage
    launches), tiny."""
    res = {}

    def put(xh, tdt):
        return torch.from_numpy(xh.view(np.int16)).to(dev).view(tdt)

    # LLaMA-3-8B prefill: the three stage launches, two buffer sets in turn
    w = synth.workload("llama3_8b_prefill")
    tdt = torch.float16 if w.dtype == synth.F16 else torch.bfloat16
    xh = synth.operands(w, seed)
    xs = [put(xh, tdt) for _ in range(2)]
    del xh
    g2 = fc.fc_stage2_group(w.R, w.H, w.group)
    bufs = [fc.fc_allreduce_emulated(x, w.bits, w.group) for x in xs]
    it = [0]

    def call8():
        i = it[0] = it[0] ^ 1
        fc.fc_allreduce_emulated(xs[i], w.bits, w.group, bufs[i][0], bufs[i][1], stream=stream)

    st = settle_clock(torch, call8, stream)
    ms = timed_calls(torch, call8, stream, 100)
    mb = model_bytes(w.R, w.T, w.H, w.bits, w.group, g2)["total"]
    res["llama3_8b_prefill"] = {
        "R": w.R, "T": w.T, "H": w.H, "io_dtype": w.dtype, "bits": w.bits, "group": w.group,
        "ms_per_step": round(ms, 6), "gbps": round(mb / (ms * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * mb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "model_bytes": mb, "steps": 100, "settle": st}
    del xs, bufs
    torch.cuda.empty_cache()

    # the group-size sweep: the same operands for every width and group length, in
    # SWEEP_SETS copies (with their own payloads and outputs) read in turn, so that a step
    # does not find its inputs in the Infinity Cache
    base = synth.workload("sweep_int4_g128")
    tdt = torch.float16 if base.dtype == synth.F16 else torch.bfloat16
    xh = synth.operands(base, seed)
    xds = [put(xh, tdt) for _ in range(SWEEP_SETS)]
    del xh
    xf = xds[0].float()
    sweep = []
    for bits in synth.SWEEP_BITS:
        for g in synth.SWEEP_GROUPS:
            R, T, H = base.R, base.T, base.H
            g2 = fc.fc_stage2_group(R, H, g)
            bufs = [fc.fc_allreduce_emulated(x, bits, g) for x in xds]
            rec = {"bits": bits, "group": g, "group2": g2}
            rec.update(stage_errors(torch, fc, xf, bufs[0][0], bufs[0][1], R, T, H, bits, bits, g, g2))
            it = [0]

            def calls(bits=bits, g=g, bufs=bufs):
                i = it[0] = (it[0] + 1) % SWEEP_SETS
                fc.fc_allreduce_emulated(xds[i], bits, g, bufs[i][0], bufs[i][1], stream=stream)

            settle_clock(torch, calls, stream, min_ms=30.0)
            ms = timed_calls(torch, calls, stream, 48)
            mb = model_bytes(R, T, H, bits, g, g2)["total"]
            rec.update({"us_per_step": round(ms * 1e3, 2), "gbps": round(mb / (ms * 1e-3) / 1e9, 1)})
            sweep.append(rec)
            del bufs
    in_mb = base.R * base.T * base.H * 2 / 1e6
    res["sweep"] = {"R": base.R, "T": base.T, "H": base.H, "io_dtype": base.dtype,
                    "note": f"{SWEEP_SETS} copies of the operands ({in_mb:.0f} MB each) with their "
                            f"own payloads, read in turn",
                    "points": sweep}
    del xds, xf
    torch.cuda.empty_cache()

    # the generic kernels: a hidden size of 5120 (not a power of two; LLaMA-2-13B's) and
    # groups of 160, which the power-of-two kernels do not take
    w = synth.workload("llama3_8b_prefill").with_(T=4096, H=5120, group=160, name="generic_h5120_g160")
    tdt = torch.float16 if w.dtype == synth.F16 else torch.bfloat16
    xh = synth.operands(w, seed)
    xds = [put(xh, tdt) for _ in range(GENERIC_SETS)]
    del xh
    bufs = [fc.fc_allreduce_emulated(x, w.bits, w.group) for x in xds]
    g2 = fc.fc_stage2_group(w.R, w.H, w.group)
    itg = [0]

    def callg():
        i = itg[0] = (itg[0] + 1) % GENERIC_SETS
        fc.fc_allreduce_emulated(xds[i], w.bits, w.group, bufs[i][0], bufs[i][1], stream=stream)

    settle_clock(torch, callg, stream, min_ms=30.0)
    ms = timed_calls(torch, callg, stream, 20)
    mb = model_bytes(w.R, w.T, w.H, w.bits, w.group, g2)["total"]
    res["generic_group"] = {"R": w.R, "T": w.T, "H": w.H, "io_dtype": w.dtype, "bits": w.bits,
                            "group": w.group, "group2": g2, "us_per_step": round(ms * 1e3, 2),
                            "gbps": round(mb / (ms * 1e-3) / 1e9, 1),
                            "note": f"generic kernels (group not a power of two); "
                                    f"{GENERIC_SETS} copies of the operands read in turn"}
    del xds, bufs
    torch.cuda.empty_cache()

    # launch-bound shapes: decode and tiny; cache-cold calls after a scratch write, and
    # back-to-back calls (the inputs then stay in the caches, as when the producing layer
    # has just written them)
    scratch = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    for name in ("decode", "tiny"):
        w = synth.workload(name)
        tdt = torch.float16 if w.dtype == synth.F16 else torch.bfloat16
        xd = put(synth.operands(w, seed), tdt)
        g2 = fc.fc_stage2_group(w.R, w.H, w.group)
        out, ws = fc.fc_allreduce_emulated(xd, w.bits, w.group)
        v = fc.workspace_views(ws, w.R, w.T, w.H, w.bits, w.group)

        def single(s=stream):
            fc.fc_allreduce_emulated(xd, w.bits, w.group, out, ws, stream=s)

        def three(s=stream):
            fc.fc_quantize_groups(xd, w.bits, w.group, v["codes1"], v["s1"], v["z1"], stream=s)
            fc.fc_dequant_sum_requant(v["codes1"], v["s1"], v["z1"], w.R, w.T, w.H, w.bits, w.group,
                                      v["codes2"], v["s2"], v["z2"], stream=s)
            fc.fc_dequantize(v["codes2"], v["s2"], v["z2"], w.T, w.H, w.bits, g2, tdt, out, stream=s)

        def noalloc(s=stream):
            fc.fc_allreduce_emulated_noalloc(xd, w.bits, w.group, out, stream=s)

        settle_clock(torch, single, stream, min_ms=30.0)
        us_single = timed_calls(torch, single, stream, 200) * 1e3
        settle_clock(torch, noalloc, stream, min_ms=30.0)
        us_noalloc = timed_calls(torch, noalloc, stream, 200) * 1e3
        us_noalloc_graph = graph_us_per_call(torch, noalloc, stream, dev)
        settle_clock(torch, three, stream, min_ms=30.0)
        us_three = timed_calls(torch, three, stream, 200) * 1e3
        us_graph = graph_us_per_call(torch, single, stream, dev)
        us_cold = cold_us_per_call(torch, single, stream, scratch)
        mb = model_bytes(w.R, w.T, w.H, w.bits, w.group, g2)["total"]
        res[name] = {"R": w.R, "T": w.T, "H": w.H, "io_dtype": w.dtype, "bits": w.bits,
                     "group": w.group, "model_bytes": mb,
                     "us_per_call_single_launch": round(us_single, 2),
                     "us_per_call_in_graph": round(us_graph, 2),
                     "us_per_call_three_launches": round(us_three, 2),
                     "us_per_call_noalloc": round(us_noalloc, 2),
                     "us_per_call_noalloc_in_graph": round(us_noalloc_graph, 2),
                     "us_per_call_cache_cold": round(us_cold, 2),
                     "gbps_single_launch": round(mb / (us_single * 1e-6) / 1e9, 1),
                     "graph_calls_per_replay": GRAPH_CALLS,
                     "timing": "HIP events around 200 back-to-back calls through the Python "
                               "binding (launch cost included), after a settle run; cache_cold: "
                               f"median of {COLD_CALLS} single launches, each timed on its own "
                               f"after a {EVICT_BYTES >> 20} MiB scratch write"}
        del xd, out, ws, v
    del scratch
    torch.cuda.empty_cache()
    return res


def stream_ceilings(torch, fc, dev, stream, nbytes: int) -> dict:
    """GB/s of the library's plain streaming kernels (the best of 1, 2, 4 and 8 loads in
    flight per lane): copy, read 4 / write 1 (K1's shape) and read only over nbytes of
    source, and read 1 / write 4 (K3's shape) over nbytes / 4 of source (nbytes written)."""
    L = fc.lib()
    probe = L.fc_internal_stream_probe
    probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                      ctypes.c_void_p]
    probe.restype = ctypes.c_int
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.random_(0, 256)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    src_bytes = {0: nbytes, 1: nbytes, 2: nbytes, 3: nbytes // 4}
    moved = {0: 2 * nbytes, 1: nbytes + nbytes // 4, 2: nbytes, 3: nbytes // 4 + nbytes}
    names = {0: "copy", 1: "read4_write1", 2: "read", 3: "read1_write4"}
    out = {}
    for kind in (0, 1, 2, 3):
        best = None
        for slots in (1, 2, 4, 8):
            def run(kind=kind, slots=slots):
                rc = probe(kind, slots, ctypes.c_void_p(src.data_ptr()),
                           ctypes.c_void_p(dst.data_ptr()), src_bytes[kind], sp)
                if rc != 0:
                    raise RuntimeError(f"fc_internal_stream_probe returned {rc}")
            settle_clock(torch, run, stream, min_ms=20.0)
            ms = timed_calls(torch, run, stream, 20)
            gbps = moved[kind] / (ms * 1e-3) / 1e9
            if best is None or gbps > best["gbps"]:
                best = {"gbps": round(gbps, 1), "slots": slots, "us": round(ms * 1e3, 2)}
        out[names[kind]] = best
    out["source_bytes"] = nbytes
    del src, dst
    torch.cuda.empty_cache()
    return out


def clock_trace(torch, fc, step, stream, dev, name: str, blocks: int = 80, per_block: int = 10,
                idle_s: float = COLD_IDLE_S) -> int:
    """From an idle GPU: `blocks` blocks of `per_block` pipeline steps back to back, the
    engine clock read with fc_internal_clock_probe after each block (a one-wave kernel,
    ~2 us), HIP events between blocks. Prints one JSON line: microseconds per step and MHz
    per block, twice (two idle starts)."""
    L = fc.lib()
    probe = L.fc_internal_clock_probe
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    probe.restype = ctypes.c_int
    buf = torch.zeros((blocks, 4), dtype=torch.int64, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    runs = []
    for rep in range(2):
        torch.cuda.synchronize()
        time.sleep(idle_s)
        ev = _events(torch, blocks + 1)
        ev[0].record(stream)
        for b in range(blocks):
            for i in range(per_block):
                step(i)
            if probe(ctypes.c_void_p(buf[b].data_ptr()), 2000, sp) != 0:
                raise RuntimeError("fc_internal_clock_probe failed")
            ev[b + 1].record(stream)
        torch.cuda.synchronize()
        c = buf.cpu()
        mhz = (c[:, 0].double() / c[:, 1].double() * 100.0).tolist()
        us = [ev[b].elapsed_time(ev[b + 1]) * 1e3 / per_block for b in range(blocks)]
        runs.append({"us_per_step": [round(u, 1) for u in us], "mhz": [round(m) for m in mhz]})
        print(f"[clock] start {rep}: first blocks " +
              " ".join(f"{u:.0f}us/{m:.0f}MHz" for u, m in zip(us[:12], mhz[:12])),
              file=sys.stderr, flush=True)
    print(json.dumps({"clock_trace": runs, "workload": name, "steps_per_block": per_block,
                      "idle_s_before": idle_s,
                      "note": "each block ends with a one-wave clock probe (~2 us), counted in "
                              "its time per step"}))
    return 0


def stage_clocks(torch, fc, step, kernel, stream, dev, name: str, n: int = 300,
                 iters: int = 500) -> None:
    """At the steady clock: n pipeline steps (buffer sets in turn, as timed) with the engine
    clock read by fc_internal_clock_probe (a one-wave kernel, ~1.5 us) before each stage
    kernel and after the last one, and HIP events around each kernel (not the probes); then
    each kernel back to back, n / 3 calls on the same buffer sets in turn. Prints one JSON
    line: median and p10 MHz at the four points, median microseconds per kernel."""
    L = fc.lib()
    probe = L.fc_internal_clock_probe
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    probe.restype = ctypes.c_int
    sp = ctypes.c_void_p(stream.cuda_stream)
    buf = torch.zeros((n, 4, 4), dtype=torch.int64, device=dev)
    it = [0]

    def one_step():
        it[0] += 1
        step(it[0])

    settle_clock(torch, one_step, stream)

    def read_clock(i, j):
        if probe(ctypes.c_void_p(buf[i, j].data_ptr()), iters, sp) != 0:
            raise RuntimeError("fc_internal_clock_probe failed")

    ev = [_events(torch, 6) for _ in range(n)]
    for i in range(n):
        for j in range(3):
            read_clock(i, j)
            ev[i][2 * j].record(stream)
            kernel(i, j)
            ev[i][2 * j + 1].record(stream)
        read_clock(i, 3)
    torch.cuda.synchronize()
    c = buf.cpu().double()
    mhz = (c[:, :, 0] / c[:, :, 1] * 100.0).tolist()
    us = [[ev[i][2 * j].elapsed_time(ev[i][2 * j + 1]) * 1e3 for j in range(3)] for i in range(n)]

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    def p10(v):
        v = sorted(v)
        return v[len(v) // 10]

    b2b = []
    for j in range(3):
        def one(j=j):
            it[0] += 1
            kernel(it[0], j)

        for _ in range(10):
            one()
        b2b.append(timed_calls(torch, one, stream, n // 3) * 1e3)
    points = ["before K1", "before K2", "before K3", "after K3"]
    print(json.dumps({"stage_clocks": {
        "workload": name, "steps": n, "probe_fma_iterations": iters,
        "mhz_median": {p: round(med([m[j] for m in mhz])) for j, p in enumerate(points)},
        "mhz_p10": {p: round(p10([m[j] for m in mhz])) for j, p in enumerate(points)},
        "us_median_in_pipeline": {k: round(med([u[j] for u in us]), 2)
                                  for j, k in enumerate(("K1", "K2", "K3"))},
        "us_back_to_back_sets_in_turn": {k: round(b2b[j], 2) for j, k in enumerate(("K1", "K2", "K3"))},
        "note": "pipeline kernels bracketed by HIP events with a clock probe before each; back "
                "to back: one kernel repeated on the buffer sets in turn"}}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the linear-layer leg (the GEMM with the quantizer in its epilogue)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline, its per-kernel pass and the streaming ceilings "
                         "(profiling runs; the ceilings' copy kernel calibrates the counters)")
    ap.add_argument("--clock-trace", action="store_true",
                    help="instead of the benchmark: from an idle GPU, run the pipeline in blocks "
                         "of 10 steps with the engine clock read after each block (the load-onset "
                         "clock dip the settle phase waits out); then, at the steady clock, the "
                         "clock at each stage boundary and each kernel's time in and out of the "
                         "pipeline")
    ap.add_argument("--quality", action="store_true",
                    help="instead of the benchmark: error (MSE) of both stages and throughput for "
                         "every block size and width of the sweep and for the five workloads")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this codec emulates the R ranks of one all-reduce on a single "
                                   "GPU; runs on more than one GPU are not supported",
                          "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import bit_activation_compression_amd as fc
    import synth

    if args.quality:
        return quality_report(args.seed)

    w = synth.workload(args.workload)
    R, T, H, bits, group = w.R, w.T, w.H, w.bits, w.group
    g2 = fc.fc_stage2_group(R, H, group)
    mb = model_bytes(R, T, H, bits, group, g2)
    tdt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] generating {w.name}: R={R} T={T} H={H} {w.dtype} int{bits} g{group}",
          file=sys.stderr, flush=True)
    x_host = synth.operands(w, args.seed)
    x_checksum = synth.checksum(x_host)

    # Two buffer sets used in turn, so a step never finds the previous step's
    # inputs or payloads in the caches.
    sets = []
    for _ in range(2):
        xd = torch.from_numpy(x_host.view(np.int16)).to(dev).view(tdt)
        c1 = torch.empty((R, T, H * bits // 8), dtype=torch.uint8, device=dev)
        s1 = torch.empty((R, T, H // group), dtype=torch.uint16, device=dev)
        z1 = torch.empty_like(s1)
        c2 = torch.empty((T, H * bits // 8), dtype=torch.uint8, device=dev)
        s2 = torch.empty((T, H // g2), dtype=torch.uint16, device=dev)
        z2 = torch.empty_like(s2)
        out = torch.empty((T, H), dtype=tdt, device=dev)
        sets.append((xd, c1, s1, z1, c2, s2, z2, out))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def kernel(i: int, j: int) -> None:
        """Kernel j (0: K1, 1: K2, 2: K3) of step i."""
        xd, c1, s1, z1, c2, s2, z2, out = sets[i % 2]
        if j == 0:
            fc.fc_quantize_groups(xd, bits, group, c1, s1, z1, stream=stream)
        elif j == 1:
            fc.fc_dequant_sum_requant(c1, s1, z1, R, T, H, bits, group, c2, s2, z2, stream=stream)
        else:
            fc.fc_dequantize(c2, s2, z2, T, H, bits, g2, tdt, out, stream=stream)

    def step(i: int, ev=None) -> None:
        for j in range(3):
            if ev is not None:
                ev[j].record(stream)
            kernel(i, j)
        if ev is not None:
            ev[3].record(stream)

    if args.clock_trace:
        rc = clock_trace(torch, fc, step, stream, dev, w.name)
        stage_clocks(torch, fc, step, kernel, stream, dev, w.name)
        return rc

    counter = [0]

    def next_step() -> None:
        step(counter[0])
        counter[0] += 1

    # 1. settle at the steady clock; 2. W warm-up steps; K timed steps, no events
    print("[bench] settling", file=sys.stderr, flush=True)
    settle = settle_clock(torch, next_step, stream)
    for i in range(args.warmup):
        step(i)
    K = args.steps
    print(f"[bench] timing {K} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # 3. per-kernel pass: events around each kernel of BREAKDOWN_STEPS steps
    events = [_events(torch, 4) for _ in range(BREAKDOWN_STEPS)]
    for i in range(BREAKDOWN_STEPS):
        step(i, ev=events[i])
    torch.cuda.synchronize()
    k_ms = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(3)] for ev in events])
    k_avg = k_ms.mean(axis=0)
    k_med = np.median(k_ms, axis=0)
    pipe_ms = np.array([ev[0].elapsed_time(ev[3]) for ev in events])

    # 4. cold start: the same K steps after the GPU has been idle
    time.sleep(COLD_IDLE_S)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - c0) * 1e3 / K

    value = mb["total"] / (ms_per_step * 1e-3) / 1e9
    k1_avg_ms = float(k_avg[0])
    k1_gbps = mb["k1"] / (k1_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "R": R, "T": T, "H": H, "io_dtype": w.dtype, "bits": bits,
                   "group": group, "group2": g2, "dist": w.dist, "sigma": w.sigma,
                   "outlier_channels": w.n_outliers, "outlier_scale": w.outlier_scale},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "elements_per_s": round(R * T * H / (ms_per_step * 1e-3), 1),
        "model_bytes": mb,
        "settle": dict(settle, note="pipeline steps run back to back before the warm-up steps "
                                    "until the time per step is steady (the GPU's power "
                                    "management lowers the engine clock for the first ~15 ms "
                                    "of load after idle)"),
        "cold_start": {"idle_s_before": COLD_IDLE_S, "ms_per_step": round(cold_ms, 6),
                       "gbps": round(mb["total"] / (cold_ms * 1e-3) / 1e9, 1),
                       "note": "the same K steps started after the GPU was idle (no settle)"},
        "breakdown_steps": BREAKDOWN_STEPS,
        "kernel_ms_avg": {"k1_quantize": round(float(k_avg[0]), 5),
                          "k2_dequant_sum_requant": round(float(k_avg[1]), 5),
                          "k3_dequantize": round(float(k_avg[2]), 5)},
        "kernel_ms_median": {"k1_quantize": round(float(k_med[0]), 5),
                             "k2_dequant_sum_requant": round(float(k_med[1]), 5),
                             "k3_dequantize": round(float(k_med[2]), 5)},
        "kernel_ms_p10_p90": {name: [round(float(np.percentile(k_ms[:, j], 10)), 5),
                                     round(float(np.percentile(k_ms[:, j], 90)), 5)]
                              for j, name in enumerate(("k1_quantize", "k2_dequant_sum_requant",
                                                        "k3_dequantize"))},
        "kernel_gbps": {"k1_quantize": round(mb["k1"] / (k_avg[0] * 1e-3) / 1e9, 1),
                        "k2_dequant_sum_requant": round(mb["k2"] / (k_avg[1] * 1e-3) / 1e9, 1),
                        "k3_dequantize": round(mb["k3"] / (k_avg[2] * 1e-3) / 1e9, 1)},
        "pipeline_ms_median_events": round(float(np.median(pipe_ms)), 5),
        "pipeline_ms_p10_p90_events": [round(float(np.percentile(pipe_ms, 10)), 5),
                                       round(float(np.percentile(pipe_ms, 90)), 5)],
        "kernel_rooflines": kernel_rooflines(mb, k_avg, w.name),
        "input_checksum": {"seed": args.seed, "blake2b_64": x_checksum},
        "link_bytes_per_rank": link_bytes(R, T, H, bits, group, g2),
        "roofline": {"bound": "hbm", "kernel": "k1_quantize", "achieved": round(k1_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(k1_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": mb["k1"],
                     "avg_launch_ms": round(k1_avg_ms, 5),
                     "timing": f"HIP events on the launch stream around K1 in each of "
                               f"{BREAKDOWN_STEPS} pipeline steps run right after the timed region "
                               f"(the bracket includes the dispatch gap before the kernel)",
                     "traffic_note": "FETCH_SIZE + WRITE_SIZE (rocprofv3) per launch, calibrated "
                                     "on a copy of known size: bytes between L2 and the data "
                                     "fabric, which count Infinity Cache hits as well as DRAM"},
    }

    print("[bench] streaming ceilings", file=sys.stderr, flush=True)
    ceil = stream_ceilings(torch, fc, dev, stream, R * T * H * 2)
    ceil["k1_frac_of_read4_write1"] = round(k1_gbps / ceil["read4_write1"]["gbps"], 4)
    ceil["k3_frac_of_read1_write4"] = round(rec["kernel_gbps"]["k3_dequantize"]
                                            / ceil["read1_write4"]["gbps"], 4)
    rec["stream_ceilings_gbps"] = ceil

    if not args.no_extras:

        # The uncompressed all-reduce result on the same operands: the arithmetic of
        # the ring all-reduce the method replaces, as an on-GPU comparator.
        xd0 = sets[0][0]
        sum_out = torch.empty((T, H), dtype=tdt, device=dev)

        def sum_call():
            fc.fc_sum_uncompressed(xd0, sum_out, stream=stream)

        settle_clock(torch, sum_call, stream, min_ms=30.0)
        sum_ms = timed_calls(torch, sum_call, stream, 50)
        sum_bytes = (R + 1) * T * H * 2
        step(0)
        torch.cuda.synchronize()
        diff = sets[0][7].float() - sum_out.float()
        mse = float((diff * diff).mean())
        ref_pow = float((sum_out.float() ** 2).mean())
        del diff
        rec["uncompressed_sum"] = {
            "ms": round(sum_ms, 5), "bytes": sum_bytes,
            "gbps": round(sum_bytes / (sum_ms * 1e-3) / 1e9, 1),
            "codec_mse_vs_uncompressed": mse,
            "codec_snr_db": round(10 * np.log10(ref_pow / mse), 2) if mse > 0 else None}

        # The residual add of the transformer block folded into the final step,
        # against the same result computed unfused (dequantize, then torch's add).
        xd0, c1, s1, z1, c2, s2, z2, out0 = sets[0]
        residual = torch.empty((T, H), dtype=tdt, device=dev).normal_(0.0, 2.0)
        res_out = torch.empty_like(residual)
        tmp = torch.empty_like(residual)

        def fused_res():
            fc.fc_dequantize_residual(c2, s2, z2, T, H, bits, g2, residual, res_out, stream=stream)

        def unfused_res():
            fc.fc_dequantize(c2, s2, z2, T, H, bits, g2, tdt, tmp, stream=stream)
            torch.add(residual, tmp, out=res_out)

        pay2 = mb["payload2"]
        settle_clock(torch, fused_res, stream, min_ms=30.0)
        res_fused_ms = timed_calls(torch, fused_res, stream, 50)
        settle_clock(torch, unfused_res, stream, min_ms=30.0)
        res_unfused_ms = timed_calls(torch, unfused_res, stream, 50)
        rec["residual_add"] = {
            "fused_ms": round(res_fused_ms, 5),
            "fused_bytes": pay2 + 2 * T * H * 2,
            "fused_gbps": round((pay2 + 2 * T * H * 2) / (res_fused_ms * 1e-3) / 1e9, 1),
            "unfused_ms": round(res_unfused_ms, 5),
            "unfused_bytes": pay2 + 4 * T * H * 2,
            "speedup": round(res_unfused_ms / res_fused_ms, 3),
        }
        del residual, res_out, tmp, sum_out

        # The row-parallel linear layers in front of the all-reduce (Figure 5,
        # left: the attention output projection o_proj, K = H / R input features
        # per rank, and the MLP down projection d_proj, K = ffn / R) with the
        # stage-1 quantization in the GEMM's epilogue, against the unfused pair
        # (torch's batched GEMM writing y, then the stage-1 kernel reading it back).
        linear = None
        if not args.no_linear:
            linear = {}
            shapes = [("o_proj", H // R)] + ([("d_proj", w.ffn // R)] if w.ffn else [])
            for name, Kl in shapes:
                if Kl % 32 or H % 256 or group > 256:
                    continue
                gen = torch.Generator(device=dev).manual_seed(args.seed)
                la = torch.randn((R, T, Kl), generator=gen, device=dev, dtype=torch.float32).to(tdt)
                lw = (torch.randn((R, H, Kl), generator=gen, device=dev, dtype=torch.float32)
                      / Kl ** 0.5).to(tdt)
                lwt = lw.transpose(1, 2).contiguous()           # [R, K, H] for torch.bmm
                ly = torch.empty((R, T, H), dtype=tdt, device=dev)

                def fused_lin():
                    fc.fc_linear_quantize(la, lw, bits, group, c1, s1, z1, stream=stream)

                def gemm_only():
                    torch.bmm(la, lwt, out=ly)

                def unfused_lin():
                    torch.bmm(la, lwt, out=ly)
                    fc.fc_quantize_groups(ly, bits, group, c1, s1, z1, stream=stream)

                flops = 2.0 * R * T * H * Kl
                n_it = max(3, min(20, int(2e13 / flops)))
                settle_clock(torch, fused_lin, stream, min_ms=30.0)
                # three rounds, the variants interleaved, median per variant: the
                # first launches after a change of shape or kernel run slower
                rounds = [[timed_calls(torch, fn, stream, n_it)
                           for fn in (fused_lin, gemm_only, unfused_lin)]
                          for _ in range(LINEAR_ROUNDS)]
                lin_ms, gemm_ms, unf_ms = (sorted(col)[len(col) // 2] for col in zip(*rounds))
                tf = flops / (lin_ms * 1e-3) / 1e12
                linear[name] = {
                    "shape": {"R": R, "T": T, "K": Kl, "H": H},
                    "fused_ms": round(lin_ms, 4),
                    "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                 "timing": f"HIP events around {n_it} back-to-back launches, median "
                                           f"of {LINEAR_ROUNDS} rounds interleaved with the "
                                           f"unfused variants"},
                    "torch_gemm_ms": round(gemm_ms, 4),
                    "torch_gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
                    "unfused_ms": round(unf_ms, 4),
                    "speedup_vs_unfused": round(unf_ms / lin_ms, 3),
                    "fusion_wins": bool(unf_ms > lin_ms),
                }
                del la, lw, lwt, ly
                torch.cuda.empty_cache()
        rec["linear_quantize"] = linear

        print("[bench] other workloads", file=sys.stderr, flush=True)
        rec["other_workloads"] = other_workloads(torch, np, fc, synth, args.seed, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print(f"[bench] timing the CPU oracle on the full workload ({CPU_PASSES} passes, 1 thread)",
              file=sys.stderr, flush=True)
        passes = []
        for _ in range(CPU_PASSES):
            c0 = time.perf_counter()
            oracle.allreduce(x_host, w.dtype, bits, group, want_f32=False)
            passes.append(time.perf_counter() - c0)
        c_s = sorted(passes)[len(passes) // 2]
        hi = host_info()
        cpu = {"value": round(mb["total"] / c_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole {w.name} workload (R={R}, T={T}, H={H}), single thread, "
                         f"median of {CPU_PASSES} passes: {c_s:.2f} s per pass "
                         f"({sum(passes):.1f} s in all) on {hi.get('model name', 'unknown')}",
               "host": hi}
    rec["cpu_baseline"] = cpu
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())

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

Prints one JSON line. `roofline` is for K1, the kernel that moves two thirds
of the bytes, timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
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


def model_bytes(R: int, T: int, H: int, bits: int, group: int, group2: int, e: int = 2) -> dict:
    n1, n2 = R * T * H, T * H
    p1 = n1 * bits // 8 + n1 // group * 4
    p2 = n2 * bits // 8 + n2 // group2 * 4
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


K1_SAMPLE_EVERY = 10
GRAPH_CALLS = 20       # calls captured per HIP graph in the launch-bound measurements
LINEAR_ROUNDS = 3      # interleaved timing rounds of the linear-layer variants
CPU_PASSES = 3         # passes of the CPU oracle over the whole workload (~4-5 s each)


def k1_sample_every(steps: int) -> int:
    """Stride of the timed steps whose K1 launch is bracketed by HIP events:
    every K1_SAMPLE_EVERY-th step, closer when that would leave fewer than 20
    samples, every step for short runs."""
    return max(1, min(K1_SAMPLE_EVERY, steps // 20))


def code_only(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed: what a
    comment edit leaves unchanged. (The kernel sources hold no string literals
    that contain comment markers.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def k1_source_hash() -> str:
    """Hash of K1's code (comments and layout ignored): the counter summary is
    valid while the code it was measured on is unchanged."""
    h = hashlib.sha256()
    for rel in K1_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str) -> float | None:
    """HBM bytes per K1 launch from the committed rocprofv3 counter summary, if it
    was taken on this workload and on the current K1 source; None otherwise."""
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def quality_report(seed: int) -> int:
    """Error of the codec at each stage, as in Figure 4 (activation quantization with blocks
    from the hidden length down to 128) and Figure 5 right (quantization before the
    Reduce-Scatter vs before the All-Gather), on the synthetic operands; plus throughput.
    The codec runs in the library's kernels; the error statistics (and the binary32
    dequantized values they need) are computed with torch on the GPU from the payloads
    the library wrote.
      stage1_mse: mean over r, t, h of (dequantized payload 1 - x)^2
      stage2_mse: mean of (dequantized payload 2 - sum_r dequantized payload 1)^2
      total_mse : mean of (output - sum_r x)^2
    Prints one JSON line with a record per configuration."""
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
        exact = xf.sum(dim=0)
        for bits, bits2 in widths[name]:
            g2 = fc.fc_stage2_group(R, H, g)
            out, ws = fc.fc_allreduce_emulated(xd, bits, g, bits2=bits2)
            v = fc.workspace_views(ws, R, T, H, bits, g, bits2=bits2)
            # the dequantized stage values in binary32, as the receiver sums them
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
            rec = {"workload": name, "bits_rs": bits, "bits_ag": bits2, "group": g, "group2": g2,
                   "stage1_mse": float(((xh32 - xf) ** 2).mean()),
                   "stage2_mse": float(((yh - y) ** 2).mean()),
                   "total_mse": float(((out.float() - exact) ** 2).mean()),
                   "exact_sum_power": float((exact ** 2).mean())}
            del s1, z1, q1, xh32, y, s2, z2, q2, yh
            # throughput of the whole path on this configuration
            for _ in range(5):
                fc.fc_allreduce_emulated(xd, bits, g, out, ws, stream=stream, bits2=bits2)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(20):
                fc.fc_allreduce_emulated(xd, bits, g, out, ws, stream=stream, bits2=bits2)
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / 20
            n1, n2 = R * T * H, T * H
            p1 = n1 * bits // 8 + n1 // g * 4
            p2 = n2 * bits2 // 8 + n2 // g2 * 4
            total = n1 * 2 + 2 * p1 + 2 * p2 + n2 * 2
            rec.update({"us_per_call": round(ms * 1e3, 2), "gbps": round(total / (ms * 1e-3) / 1e9, 1)})
            if T * H <= 1 << 20:
                # launch-bound shapes: GRAPH_CALLS consecutive calls captured in one
                # HIP graph (as a serving step would be) and replayed; per-call time
                graph = torch.cuda.CUDAGraph()
                cap = torch.cuda.Stream(dev)
                cap.wait_stream(stream)
                with torch.cuda.stream(cap):
                    fc.fc_allreduce_emulated(xd, bits, g, out, ws, stream=cap, bits2=bits2)
                    with torch.cuda.graph(graph, stream=cap):
                        for _ in range(GRAPH_CALLS):
                            fc.fc_allreduce_emulated(xd, bits, g, out, ws, stream=cap, bits2=bits2)
                stream.wait_stream(cap)
                torch.cuda.synchronize()
                for _ in range(3):
                    graph.replay()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record(stream)
                for _ in range(10):
                    graph.replay()
                ev[1].record(stream)
                torch.cuda.synchronize()
                rec["us_per_call_graph"] = round(ev[0].elapsed_time(ev[1]) / (10 * GRAPH_CALLS) * 1e3, 2)
                rec["graph_calls_per_replay"] = GRAPH_CALLS
                del graph
            records.append(rec)
            print(f"[quality] {name} int{bits}->int{bits2}: stage1 {rec['stage1_mse']:.4g} "
                  f"stage2 {rec['stage2_mse']:.4g} total {rec['total_mse']:.4g} "
                  f"{rec['us_per_call']} us {rec['gbps']} GB/s", file=sys.stderr, flush=True)
        del xd, xf, exact
    print(json.dumps({"quality": records, "seed": seed, "data": "synthetic"}))
    return 0


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

    def step(i: int, k1_ev=None, all_ev=None) -> None:
        xd, c1, s1, z1, c2, s2, z2, out = sets[i % 2]
        if k1_ev is not None:
            k1_ev[0].record(stream)
        if all_ev is not None:
            all_ev[0].record(stream)
        fc.fc_quantize_groups(xd, bits, group, c1, s1, z1, stream=stream)
        if k1_ev is not None:
            k1_ev[1].record(stream)
        if all_ev is not None:
            all_ev[1].record(stream)
        fc.fc_dequant_sum_requant(c1, s1, z1, R, T, H, bits, group, c2, s2, z2, stream=stream)
        if all_ev is not None:
            all_ev[2].record(stream)
        fc.fc_dequantize(c2, s2, z2, T, H, bits, g2, tdt, out, stream=stream)
        if all_ev is not None:
            all_ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps. The only events in it bracket K1, the kernel
    # whose roofline is reported, on a sample of the steps (every
    # K1_SAMPLE_EVERY-th, at least 20 of them when K allows): each event is a
    # packet in the stream that adds a few microseconds between kernels, so
    # bracketing every launch would slow the whole step down. The K2/K3 split
    # is timed separately below.
    K = args.steps
    every = k1_sample_every(K)
    k1_events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                 for i in range(0, K, every)}
    print(f"[bench] timing {K} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, k1_ev=k1_events.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    k1_ms = np.array([ev[0].elapsed_time(ev[1]) for ev in k1_events.values()])

    # Per-kernel breakdown (not part of the timed region).
    KB = min(K, 50)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(KB)]
    for i in range(KB):
        step(i, all_ev=events[i])
    torch.cuda.synchronize()
    k_ms = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(3)] for ev in events])
    k_avg = k_ms.mean(axis=0)
    k_med = np.median(k_ms, axis=0)
    pipe_ms = np.array([ev[0].elapsed_time(ev[3]) for ev in events])

    # a plain device-to-device copy of 1 GiB: the runtime's own streaming kernel
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(10):
        dst.copy_(src)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src, dst

    # The uncompressed all-reduce result on the same operands: the arithmetic of
    # the ring all-reduce the method replaces, as an on-GPU comparator.
    xd0 = sets[0][0]
    sum_out = torch.empty((T, H), dtype=tdt, device=dev)
    for _ in range(5):
        fc.fc_sum_uncompressed(xd0, sum_out, stream=stream)
    se = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    se[0].record(stream)
    for _ in range(50):
        fc.fc_sum_uncompressed(xd0, sum_out, stream=stream)
    se[1].record(stream)
    torch.cuda.synchronize()
    sum_ms = se[0].elapsed_time(se[1]) / 50
    sum_bytes = (R + 1) * T * H * 2
    # codec output vs the uncompressed result (diagnostic, in torch on the GPU)
    step(0)
    torch.cuda.synchronize()
    diff = sets[0][7].float() - sum_out.float()
    mse = float((diff * diff).mean())
    ref_pow = float((sum_out.float() ** 2).mean())
    del diff

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

    def timed(fn, n=50):
        for _ in range(5):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(n):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    pay2 = T * H * bits // 8 + T * (H // g2) * 4
    res_fused_ms = timed(fused_res)
    res_unfused_ms = timed(unfused_res)
    residual_add = {
        "fused_ms": round(res_fused_ms, 5),
        "fused_bytes": pay2 + 2 * T * H * 2,
        "fused_gbps": round((pay2 + 2 * T * H * 2) / (res_fused_ms * 1e-3) / 1e9, 1),
        "unfused_ms": round(res_unfused_ms, 5),
        "unfused_bytes": pay2 + 4 * T * H * 2,
        "speedup": round(res_unfused_ms / res_fused_ms, 3),
    }
    del residual, res_out, tmp

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
            # three rounds, the variants interleaved, median per variant: the
            # first launches after a change of shape or kernel run slower
            rounds = [[timed(fn, n_it) for fn in (fused_lin, gemm_only, unfused_lin)]
                      for _ in range(LINEAR_ROUNDS)]
            lin_ms, gemm_ms, unf_ms = (sorted(col)[len(col) // 2] for col in zip(*rounds))
            tf = flops / (lin_ms * 1e-3) / 1e12
            linear[name] = {
                "shape": {"R": R, "T": T, "K": Kl, "H": H},
                "fused_ms": round(lin_ms, 4),
                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                             "timing": f"HIP events around {n_it} back-to-back launches, median of "
                                       f"{LINEAR_ROUNDS} rounds interleaved with the unfused variants"},
                "torch_gemm_ms": round(gemm_ms, 4),
                "torch_gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
                "unfused_ms": round(unf_ms, 4),
                "speedup_vs_unfused": round(unf_ms / lin_ms, 3),
            }
            del la, lw, lwt, ly
            torch.cuda.empty_cache()

    value = mb["total"] / (ms_per_step * 1e-3) / 1e9
    k1_avg_ms = float(k1_ms.mean())
    k1_gbps = mb["k1"] / (k1_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)

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
        cpu = {"value": round(mb["total"] / c_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole {w.name} workload (R={R}, T={T}, H={H}), single thread, "
                         f"median of {CPU_PASSES} passes: {c_s:.2f} s per pass "
                         f"({sum(passes):.1f} s in all) on {cpu_model()}"}

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
        "breakdown_steps": KB,
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
        "input_checksum": {"seed": args.seed, "blake2b_64": x_checksum},
        "copy_ceiling_gbps": round(copy_gbps, 1),
        "uncompressed_sum": {"ms": round(sum_ms, 5), "bytes": sum_bytes,
                             "gbps": round(sum_bytes / (sum_ms * 1e-3) / 1e9, 1),
                             "codec_mse_vs_uncompressed": mse,
                             "codec_snr_db": round(10 * np.log10(ref_pow / mse), 2) if mse > 0 else None},
        "link_bytes_per_rank": link_bytes(R, T, H, bits, group, g2),
        "residual_add": residual_add,
        "linear_quantize": linear,
        "roofline": {"bound": "hbm", "kernel": "k1_quantize", "achieved": round(k1_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(k1_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": mb["k1"],
                     "avg_launch_ms": round(k1_avg_ms, 5),
                     "timing": f"HIP events around the K1 launch of one timed step in {every} "
                               f"({len(k1_ms)} launches)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())

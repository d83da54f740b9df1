"""Seeded random shapes through the C ABI against the CPU oracle.

Method: "Flash Communication: ..." (Figure 5, right; Figure 3 for the
residual add). The shapes are drawn to cover the library's dispatch space: R
from 1 to 8 (compile-time and run-time operand counts), every group length
from 8 to 8192 with groups inside a lane run, across lanes and across wave
slots, stage-2 groups equal to or shorter than the stage-1 groups (group >
H/R), both code widths before each step, both dtypes, with and without the
residual add, and both the single-launch and the three-launch paths of
fc_allreduce_emulated. Bar: payloads and output bit-exact.

Also: calls on two streams at once give the same bits as calls one at a time
(the header promises no global state).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle
import synth

pytestmark = pytest.mark.gpu

TDT = {synth.F16: torch.float16, synth.BF16: torch.bfloat16}
PAYLOAD = ("codes1", "s1", "z1", "codes2", "s2", "z2")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    fc.lib()
    yield


def _dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(TDT[dtype])


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype in (torch.uint16, torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _draw(rng) -> tuple:
    """A valid (R, T, H, group, bits, bits2, dtype, residual) with T*H small."""
    while True:
        R = int(rng.integers(1, 9))
        group = int(2 ** rng.integers(3, 14))                # 8 .. 8192
        # stage-2 group: the group itself, or the chunk when the group is longer
        if rng.random() < 0.75:
            g2 = group
            C = g2 * int(rng.integers(1, 5))
        else:
            C = int(2 ** rng.integers(3, 14))
            if C >= group:
                continue
            g2 = C
        H = R * C
        if H % group or H > 32768:
            continue
        if oracle.stage2_group(R, H, group) != g2:
            continue
        T = int(rng.integers(1, max(2, min(40, (1 << 19) // H))))
        bits, bits2 = int(rng.choice([4, 8])), int(rng.choice([4, 8]))
        dtype = synth.F16 if rng.random() < 0.5 else synth.BF16
        return R, T, H, group, bits, bits2, dtype, bool(rng.random() < 0.3)


CASES = [_draw(np.random.default_rng(2024 + i)) for i in range(100)]


@pytest.mark.parametrize("case", CASES, ids=[f"R{c[0]}T{c[1]}H{c[2]}g{c[3]}b{c[4]}{c[5]}{c[6]}{'r' if c[7] else ''}"
                                             for c in CASES])
def test_random_shape(case):
    R, T, H, group, bits, bits2, dtype, with_res = case
    print(f"[gpu] random shape R={R} T={T} H={H} g={group} int{bits}->int{bits2} {dtype} "
          f"residual={with_res}", file=sys.stderr, flush=True)
    w = synth.workload("tiny").with_(name="random", R=R, T=T, H=H, bits=bits, group=group, dtype=dtype,
                                     outlier_frac=0.02, outlier_scale=25.0)
    x = synth.operands(w, R * 1000 + T)
    ref = oracle.allreduce(x, dtype, bits, group, want_f32=False, bits2=bits2)
    res = None
    if with_res:
        v = np.random.default_rng(T + H).standard_normal((T, H))
        res = oracle.float_to_half(v) if dtype == synth.F16 else oracle.float_to_bf16(v)
        ref["out"] = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], T, H, bits2,
                                                ref["group2"], dtype, res)
    out, ws = fc.fc_allreduce_emulated(_dev(x, dtype), bits, group, bits2=bits2,
                                       residual=None if res is None else _dev(res, dtype))
    views = fc.workspace_views(ws, R, T, H, bits, group, bits2=bits2)
    torch.cuda.synchronize()
    got = {k: _np(v) for k, v in views.items()}
    got["out"] = _np(out)
    for k in PAYLOAD + ("out",):
        a, b = np.asarray(got[k]).reshape(-1), np.asarray(ref[k]).reshape(-1)
        assert np.array_equal(a, b), f"{k}: {np.count_nonzero(a != b)} of {a.size} differ"


def test_two_streams_at_once():
    """Two different calls in flight on two streams give the bits each gives
    alone."""
    # the first takes the three launches, the second the single launch
    shapes = [(4, 2048, 4096, 128, 4, synth.BF16), (8, 64, 8192, 128, 4, synth.BF16)]
    inputs, alone = [], []
    for (R, T, H, g, b, dt) in shapes:
        w = synth.workload("tiny").with_(name="streams", R=R, T=T, H=H, bits=b, group=g, dtype=dt)
        xd = _dev(synth.operands(w, T), dt)
        out, ws = fc.fc_allreduce_emulated(xd, b, g)
        torch.cuda.synchronize()
        inputs.append((xd, b, g))
        alone.append((out.clone(), ws.clone()))

    def payloads(ws, i):
        R, T, H, g, b, _ = shapes[i]
        return [v.clone() for v in fc.workspace_views(ws, R, T, H, b, g).values()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(a[0]) for a in alone]
    wss = [torch.empty_like(a[1]) for a in alone]
    torch.cuda.synchronize()
    for _ in range(10):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                xd, b, g = inputs[i]
                fc.fc_allreduce_emulated(xd, b, g, outs[i], wss[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(outs[i], alone[i][0]), f"stream {i}: output"
        for a, b in zip(payloads(wss[i], i), payloads(alone[i][1], i)):
            assert torch.equal(a, b), f"stream {i}: payload"


def test_host_threads_at_once():
    """Four host threads, each on its own stream, calling the library together (the
    binding releases the interpreter lock during each call): the per-device caches the
    library keeps (compute units, its allocation-free scratch address) are filled by
    whichever call comes first, and every call gives the bits it gives alone. The
    calls cover the three launches, the single launch, the linear layer and the
    generic kernels; the allocation-free entry point runs on one thread only, since
    overlapping calls of it on one device share its scratch."""
    import threading

    cases = [
        ("steps", (4, 2048, 4096, 128, 4, synth.BF16)),
        ("single", (8, 64, 8192, 128, 4, synth.BF16)),
        ("generic", (4, 512, 5120, 160, 4, synth.F16)),
        ("noalloc", (2, 256, 2048, 64, 8, synth.F16)),
    ]
    work = []
    for name, (R, T, H, g, b, dt) in cases:
        w = synth.workload("tiny").with_(name="threads", R=R, T=T, H=H, bits=b, group=g, dtype=dt)
        xd = _dev(synth.operands(w, H + T), dt)
        want, _ = fc.fc_allreduce_emulated(xd, b, g)
        work.append((name, xd, b, g, want))
    # the linear layer too, with its own compute-unit lookup
    rng = np.random.default_rng(31)
    la = synth.operands_from_values(rng.normal(size=(2, 300, 512)), synth.BF16)
    lw = synth.operands_from_values(rng.normal(size=(2, 1024, 512)) * 0.05, synth.BF16)
    la_d, lw_d = _dev(la, synth.BF16), _dev(lw, synth.BF16)
    lin_want = fc.fc_linear_quantize(la_d, lw_d, 4, 128)
    torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            name, xd, b, g, want = work[i]
            with torch.cuda.stream(s):
                for _ in range(8):
                    if name == "noalloc":
                        out = fc.fc_allreduce_emulated_noalloc(xd, b, g)
                    else:
                        out, _ = fc.fc_allreduce_emulated(xd, b, g)
                    lin = fc.fc_linear_quantize(la_d, lw_d, 4, 128)
            s.synchronize()
            if not torch.equal(out, want):
                errors.append(f"{name}: output")
            for a, c in zip(lin, lin_want):
                if a is not None and not torch.equal(a, c):
                    errors.append(f"{name}: linear payload")
        except Exception as e:   # reported below, from the main thread
            errors.append(f"{work[i][0]}: {e!r}")

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(work))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors

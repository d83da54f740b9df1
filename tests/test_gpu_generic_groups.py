"""GPU parity for group lengths that are not a power of two in [8, 8192]: the
generic kernels (csrc/fc_generic.hip) through the C ABI, bit-exact against
the CPU oracle on both payloads and the output.

The boundary takes any even group length dividing H whose stage-2 group
g2 = min(group, H/R) is even and divides H/R: "Flash Communication: Reducing
Tensor Parallelization Bottleneck for Fast Large Language Model Inference",
Figure 4 (block-wise quantization along the hidden dimension) and Figure 5,
right (quantization before the Reduce-Scatter and before the All-Gather).
Cases cover both lane units (8 values when the group lengths are multiples
of 8, else 2) in both layouts (groups of at most 64 units sharing a wave,
longer groups one per wave), mixed units between the two stages,
power-of-two groups below 8 and above 8192, stage-1 groups on the fast
kernel with a stage-2 group on the generic one, mixed widths, ragged token counts, R = 1 .. 8, the residual add, edge
values, T = 0, and a random sample of shapes. Inputs: the seeded generator.
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


def _say(msg: str) -> None:
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype in (torch.uint16, torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x.view(np.int16)).cuda().view(TDT[dtype])


def _workload(R, T, H, bits, g, dtype, src="llama3_8b_prefill"):
    return synth.workload(src).with_(R=R, T=T, H=H, bits=bits, group=g, dtype=dtype,
                                     name=f"R{R}_T{T}_H{H}_int{bits}_g{g}_{dtype}")


def _compare(got: dict, ref: dict, label: str) -> None:
    for k in PAYLOAD + ("out",):
        a = np.asarray(got[k]).reshape(-1)
        b = np.asarray(ref[k]).reshape(-1)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{label}: {k} differs at {bad.size} of {a.size}, first "
                                 f"{bad[:6]}: got {a[bad[:6]]} want {b[bad[:6]]}")


def _allreduce(x, dtype, bits, g, bits2=None):
    R, T, H = x.shape
    out, ws = fc.fc_allreduce_emulated(_dev(x, dtype), bits, g, bits2=bits2)
    v = fc.workspace_views(ws, R, T, H, bits, g, bits2=bits2)
    torch.cuda.synchronize()
    got = {k: _np(t) for k, t in v.items()}
    got["out"] = _np(out)
    return got


def _steps(x, dtype, bits, g, bits2=None):
    R, T, H = x.shape
    b2 = bits if bits2 is None else bits2
    c1, s1, z1 = fc.fc_quantize_groups(_dev(x, dtype), bits, g)
    c2, s2, z2 = fc.fc_dequant_sum_requant(c1, s1, z1, R, T, H, bits, g, bits2=b2)
    g2 = fc.fc_stage2_group(R, H, g)
    out = fc.fc_dequantize(c2, s2, z2, T, H, b2, g2, TDT[dtype])
    torch.cuda.synchronize()
    return {k: _np(t) for k, t in zip(PAYLOAD + ("out",), (c1, s1, z1, c2, s2, z2, out))}


CASES = [  # R, T, H, bits1, bits2, group, dtype
    (2, 8, 12, 4, 4, 2, synth.F16),          # the smallest group
    (2, 5, 24, 8, 8, 6, synth.BF16),         # 3 pairs in a 4-lane segment
    (4, 16, 96, 4, 4, 24, synth.F16),        # groups = chunks of 24
    (3, 7, 576, 8, 4, 96, synth.F16),        # R = 3, mixed widths
    (4, 9, 4608, 4, 8, 96, synth.BF16),      # mixed widths, many groups per row
    (5, 6, 600, 4, 4, 40, synth.BF16),       # R = 5
    (4, 33, 1536, 8, 8, 192, synth.BF16),    # 96 pairs: one group per wave
    (8, 4, 1920, 4, 4, 240, synth.F16),      # R = 8, chunk of 240
    (4, 3, 6144, 4, 4, 6144, synth.F16),     # group over chunks: stage 2 on 1536
    (4, 5, 384, 4, 4, 128, synth.F16),       # stage 1 fast (128), stage 2 generic (96)
    (2, 8, 256, 4, 4, 4, synth.BF16),        # power of two below 8
    (1, 2, 16384, 4, 4, 16384, synth.F16),   # power of two above 8192, R = 1
    (4, 1, 6144, 8, 8, 3072, synth.BF16),    # g > C = 1536, one token
    (6, 11, 1152, 4, 4, 12, synth.F16),      # R = 6, ragged tokens
    (4, 5, 48, 4, 4, 24, synth.F16),         # stage 1 in octets, stage 2 (12) in pairs
    (4, 3, 48, 8, 4, 16, synth.BF16),        # stage 1 fast (16), stage 2 (12) in pairs
    (3, 4, 24, 4, 8, 12, synth.F16),         # stage 1 in pairs, stage 2 fast (8)
    (2, 7, 1040, 8, 8, 520, synth.BF16),     # 65 octets: one group per wave
    (4, 6, 448, 4, 4, 56, synth.F16),        # units of 7 vectors, one lane per group
    (2, 5, 2240, 8, 4, 224, synth.BF16),     # units of 7 vectors, 4 lanes per group
    (2, 3, 10240, 4, 4, 5120, synth.F16),    # units of 5 vectors, one group per wave
    (1, 2, 7168, 8, 8, 7168, synth.BF16),    # units of 7 vectors, one group per wave
    (4, 9, 2560, 4, 4, 160, synth.BF16),     # units of 5 vectors, 4 lanes per group
    (16, 4, 1536, 4, 4, 96, synth.F16),      # R = 16: the reduction's run-time operand loop
    (24, 3, 2304, 8, 4, 96, synth.BF16),     # R = 24, mixed widths
    (12, 5, 1440, 4, 4, 120, synth.F16),     # R = 12, units of 1 vector (15 of 16 lanes)
    # groups of at most 32 values, not a multiple of 8: a lane owns a group in stage 1
    (4, 37, 1280, 4, 4, 10, synth.F16),      # 296 full waves of groups
    (3, 13, 420, 8, 8, 14, synth.BF16),      # INT8, a partial last wave
    (2, 9, 960, 4, 8, 30, synth.F16),        # the longest such group, mixed widths
    (5, 3, 3200, 8, 4, 10, synth.BF16),      # R = 5
    (4, 6, 2080, 4, 4, 26, synth.F16),       # 13 pairs per lane
]


@pytest.mark.parametrize("R,T,H,b1,b2,g,dt", CASES)
def test_generic_groups_bit_exact(R, T, H, b1, b2, g, dt):
    w = _workload(R, T, H, b1, g, dt)
    assert fc.fc_stage2_group(R, H, g) > 0
    _say(f"generic {w.name} bits2={b2}")
    x = synth.operands(w, 7)
    ref = oracle.allreduce(x, dt, b1, g, want_f32=False, bits2=b2)
    _compare(_allreduce(x, dt, b1, g, bits2=b2), ref, w.name)
    _compare(_steps(x, dt, b1, g, bits2=b2), ref, w.name + " (three entry points)")


def test_generic_groups_larger_shape():
    # 70B-like operands with groups of 96 (non power of two), 1024 tokens
    w = _workload(4, 1024, 4608, 4, 96, synth.BF16, src="llama3_70b_prefill")
    _say(f"generic {w.name}")
    x = synth.operands(w, 2)
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    _compare(_allreduce(x, w.dtype, w.bits, w.group), ref, w.name)


def test_generic_groups_edge_values():
    """Constant groups, signed zeros, fp16 subnormals, large magnitudes (groups of 24)."""
    R, T, H, g = 2, 6, 96, 24
    rng = np.random.default_rng(4)
    v = rng.standard_normal((R, T, H)).astype(np.float32)
    v[:, 0] = 1.5
    v[:, 1, ::2] = -0.0
    v[:, 1, 1::2] = 0.0
    v[:, 2] *= 1e-6
    v[:, 3] *= 3000.0
    v[0, 4, :24] = 7.0
    for dt in (synth.F16, synth.BF16):
        x = synth.operands_from_values(v, dt)
        for bits in (4, 8):
            ref = oracle.allreduce(x, dt, bits, g, want_f32=False)
            _compare(_allreduce(x, dt, bits, g), ref, f"edge {dt} int{bits}")


def test_generic_groups_residual():
    R, T, H, g = 3, 10, 576, 96
    for dt in (synth.F16, synth.BF16):
        for bits, bits2 in ((4, 4), (8, 4), (4, 8)):
            w = _workload(R, T, H, bits, g, dt)
            x = synth.operands(w, 3)
            rng = np.random.default_rng(9)
            res = synth.operands_from_values(rng.standard_normal((T, H)).astype(np.float32) * 3, dt)
            ref = oracle.allreduce(x, dt, bits, g, want_f32=False, bits2=bits2)
            g2 = ref["group2"]
            want = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], T, H, bits2, g2,
                                              dt, res)
            rd = _dev(res, dt)
            out, _ = fc.fc_allreduce_emulated(_dev(x, dt), bits, g, bits2=bits2, residual=rd)
            torch.cuda.synchronize()
            assert np.array_equal(_np(out), want), (dt, bits, bits2)
            # the stage entry point, in place on the residual
            c2 = torch.from_numpy(np.ascontiguousarray(ref["codes2"])).cuda()
            s2 = torch.from_numpy(ref["s2"].view(np.int16)).cuda().view(torch.uint16)
            z2 = torch.from_numpy(ref["z2"].view(np.int16)).cuda().view(torch.uint16)
            fc.fc_dequantize_residual(c2, s2, z2, T, H, bits2, g2, rd, out=rd)
            torch.cuda.synchronize()
            assert np.array_equal(_np(rd), want), (dt, bits, bits2, "in place")


def test_generic_groups_no_tokens():
    x = torch.empty((3, 0, 576), dtype=torch.float16, device="cuda")
    out, _ = fc.fc_allreduce_emulated(x, 4, 96)
    assert out.shape == (0, 576)
    c1, s1, z1 = fc.fc_quantize_groups(x, 4, 96)
    assert c1.shape == (3, 0, 288) and s1.shape == (3, 0, 6)


def test_generic_groups_random_shapes():
    rng = np.random.default_rng(2026)
    done = 0
    while done < 40:
        R = int(rng.integers(1, 9))
        g = 2 * int(rng.integers(1, 400))
        k = int(rng.integers(1, 6))
        H = g * k
        if H % R or H > 20000:
            continue
        C = H // R
        g2 = min(g, C)
        if g2 % 2 or C % g2:
            continue
        if fc.fc_stage2_group(R, H, g) != g2:
            raise AssertionError((R, H, g))
        T = int(rng.integers(1, 40))
        b1, b2 = int(rng.choice([4, 8])), int(rng.choice([4, 8]))
        dt = synth.F16 if rng.integers(0, 2) else synth.BF16
        w = _workload(R, T, H, b1, g, dt, src="decode" if done % 3 == 0 else "llama3_8b_prefill")
        x = synth.operands(w, done)
        ref = oracle.allreduce(x, dt, b1, g, want_f32=False, bits2=b2)
        _compare(_allreduce(x, dt, b1, g, bits2=b2), ref, f"random {w.name} bits2={b2}")
        done += 1
    _say(f"generic random shapes: {done} bit-exact")

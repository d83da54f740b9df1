"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Method: "Flash Communication: Reducing Tensor Parallelization Bottleneck for
Fast Large Language Model Inference" (Figure 4; Figure 5, right).

Bar: codes, scales and zeros of both payloads bit-exact; the output within
|out - ref| <= sum_r s1_r/2 + s2/2 + 2^-10 |ref| (ref = the oracle's output),
and in fact expected bit-exact because every rounding step is the same.
Inputs come from the seeded generator (synth), never from the GPU.
"""
from __future__ import annotations

import functools
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    fc.lib()
    yield


@functools.lru_cache(maxsize=4)
def _case(w: synth.Workload, seed: int):
    x = synth.operands(w, seed)
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    return x, ref


def _to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x.view(np.int16)).cuda().view(TDT[dtype])


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype in (torch.uint16, torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _run_fused(x: np.ndarray, w: synth.Workload, bits2: int | None = None) -> dict:
    R, T, H = x.shape
    xd = _to_dev(x, w.dtype)
    out, ws = fc.fc_allreduce_emulated(xd, w.bits, w.group, bits2=bits2)
    views = fc.workspace_views(ws, R, T, H, w.bits, w.group, bits2=bits2)
    torch.cuda.synchronize()
    got = {k: _np(v) for k, v in views.items()}
    got["out"] = _np(out)
    return got


def _run_steps(x: np.ndarray, w: synth.Workload, bits2: int | None = None) -> dict:
    R, T, H = x.shape
    b2 = w.bits if bits2 is None else bits2
    xd = _to_dev(x, w.dtype)
    c1, s1, z1 = fc.fc_quantize_groups(xd, w.bits, w.group)
    c2, s2, z2 = fc.fc_dequant_sum_requant(c1, s1, z1, R, T, H, w.bits, w.group, bits2=b2)
    g2 = fc.fc_stage2_group(R, H, w.group)
    out = fc.fc_dequantize(c2, s2, z2, T, H, b2, g2, TDT[w.dtype])
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in zip(PAYLOAD + ("out",), (c1, s1, z1, c2, s2, z2, out))}


def _widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == synth.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check(got: dict, ref: dict, w: synth.Workload, x: np.ndarray, rows=None) -> None:
    R, T, H = x.shape
    for k in PAYLOAD:
        a = np.asarray(got[k]).reshape(-1)
        b = np.asarray(ref[k]).reshape(-1)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{w.name}: {k} differs at {bad.size} of {a.size} positions, "
                                 f"first {bad[:8]}: got {a[bad[:8]]} want {b[bad[:8]]}")
    # the stated tolerance on the output, on all rows or on a sample of rows
    rows = np.arange(T) if rows is None else rows
    g2 = ref["group2"]
    s1 = ref["s1"].reshape(R, T, -1)[:, rows].view(np.float16).astype(np.float64)
    s2 = ref["s2"].reshape(T, -1)[rows].view(np.float16).astype(np.float64)
    tol = (np.repeat(s1, w.group, axis=2).sum(axis=0) / 2 + np.repeat(s2, g2, axis=1) / 2)
    want = _widen(ref["out"].reshape(T, H)[rows], w.dtype)
    have = _widen(got["out"].reshape(T, H)[rows], w.dtype)
    tol = tol + 2.0 ** -10 * np.abs(want)
    assert np.all(np.abs(have - want) <= tol), f"{w.name}: output outside the tolerance"
    assert np.array_equal(np.asarray(got["out"]).reshape(-1), np.asarray(ref["out"]).reshape(-1)), \
        f"{w.name}: output within tolerance but not bit-exact"


# ---------------------------------------------------------------------------
# the five workloads at their full sizes
# ---------------------------------------------------------------------------

FULL = ["tiny", "llama3_8b_prefill", "llama3_70b_prefill", "decode"] + [
    f"sweep_int{b}_g{g}" for b in synth.SWEEP_BITS for g in synth.SWEEP_GROUPS]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size(name):
    w = synth.workload(name)
    x, ref = _case(w, 0)
    _say(f"{name} R={w.R} T={w.T} H={w.H} bits={w.bits} group={w.group} seed=0 fused")
    got = _run_fused(x, w)
    rows = None if w.T <= 512 else np.random.default_rng(0).choice(w.T, 256, replace=False)
    _check(got, ref, w, x, rows)


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["llama3_8b_prefill", "decode"])
def test_more_seeds(name, seed):
    w = synth.workload(name)
    x, ref = _case(w, seed)
    _say(f"{name} seed={seed} separate entry points")
    got = _run_steps(x, w)
    rows = None if w.T <= 512 else np.random.default_rng(seed).choice(w.T, 256, replace=False)
    _check(got, ref, w, x, rows)


def test_tiny_many_seeds():
    w = synth.workload("tiny")
    _say("tiny seeds 0..99")
    for seed in range(100):
        x = synth.operands(w, seed)
        ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
        _check(_run_fused(x, w), ref, w, x)


# ---------------------------------------------------------------------------
# ragged shapes, every group length, R from 1 to 8, tails inside a slot
# ---------------------------------------------------------------------------

RAGGED = [
    # R, T, H, bits, group, dtype
    (1, 5, 64, 4, 64, synth.F16),
    (2, 17, 32, 4, 16, synth.BF16),
    (2, 33, 1024, 8, 8, synth.F16),
    (3, 7, 384, 4, 128, synth.BF16),
    (5, 3, 640, 8, 128, synth.F16),
    (6, 11, 3072, 4, 512, synth.BF16),
    (7, 5, 7168, 4, 1024, synth.F16),
    (8, 9, 8192, 4, 8192, synth.BF16),
    (4, 1, 16384, 8, 4096, synth.F16),
    (1, 3, 8192, 8, 2048, synth.BF16),
    (4, 13, 4096, 4, 32, synth.F16),
    (2, 3, 2048, 8, 256, synth.BF16),
    (8, 2, 1024, 4, 128, synth.F16),
    (4, 129, 4096, 8, 4096, synth.BF16),
    # n = T*H not a multiple of 32: the last lane's run of 32 positions ends
    # after 8, 16 or 24 of them (stage-2 groups of 8 or 16)
    (1, 3, 40, 4, 8, synth.F16),
    (1, 3, 48, 8, 16, synth.BF16),
    (2, 5, 48, 4, 8, synth.BF16),
    (2, 5, 48, 8, 8, synth.F16),
    (3, 3, 24, 8, 8, synth.F16),
    # stage-2 groups of 8192: one group spans four wave slots
    (1, 2, 8192, 4, 8192, synth.F16),
    (2, 3, 16384, 8, 8192, synth.BF16),
]


@pytest.mark.parametrize("R,T,H,bits,group,dtype", RAGGED)
def test_ragged_shapes(R, T, H, bits, group, dtype):
    w = synth.workload("tiny").with_(name="ragged", R=R, T=T, H=H, bits=bits, group=group,
                                     dtype=dtype, outlier_frac=0.01, outlier_scale=20.0)
    x = synth.operands(w, 7)
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    _say(f"ragged R={R} T={T} H={H} bits={bits} group={group} {dtype}")
    _check(_run_fused(x, w), ref, w, x)
    _check(_run_steps(x, w), ref, w, x)


# more operands than the compile-time reduction paths (2, 4, 8) and the
# single-launch path (up to 8) take: the reduction's run-time operand loop
MANY = [
    # R, T, H, bits, group, dtype
    (12, 5, 1536, 8, 64, synth.F16),
    (16, 7, 2048, 4, 128, synth.BF16),
    (32, 3, 4096, 4, 128, synth.F16),
    (64, 2, 8192, 8, 128, synth.BF16),
    (16, 3, 512, 4, 32, synth.F16),
]


@pytest.mark.parametrize("R,T,H,bits,group,dtype", MANY)
def test_many_operands(R, T, H, bits, group, dtype):
    w = synth.workload("tiny").with_(name="many", R=R, T=T, H=H, bits=bits, group=group,
                                     dtype=dtype, outlier_frac=0.01, outlier_scale=20.0)
    x = synth.operands(w, 11)
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    _say(f"many operands R={R} T={T} H={H} bits={bits} group={group} {dtype}")
    _check(_run_fused(x, w), ref, w, x)
    _check(_run_steps(x, w), ref, w, x)


def test_empty_token_dimension():
    x = torch.empty((4, 0, 512), dtype=torch.float16, device="cuda")
    out, ws = fc.fc_allreduce_emulated(x, 4, 128)
    torch.cuda.synchronize()
    assert out.shape == (0, 512)


# ---------------------------------------------------------------------------
# hand-built edge groups
# ---------------------------------------------------------------------------

def _edge_values(dtype: str) -> np.ndarray:
    """R=4, T=8, H=512, groups of 128: constant, signed zeros, exact ramps,
    subnormals, a stage-2 bottom clamp, large magnitudes, alternating signs."""
    R, T, H = 4, 8, 512
    rng = np.random.default_rng(5)
    v = np.zeros((R, T, H))
    v[:, 0] = np.repeat(rng.integers(-16, 16, size=(R, H // 128)) / 8.0, 128, axis=1)   # constant
    v[:, 1] = 0.0                                                                    # zeros (signs below)
    v[:, 2] = (np.arange(H) % 16) / 16.0 - 0.5                                        # ramps
    v[:, 3] = (np.arange(H) % 22) * 2.0 ** -24                                        # fp16 subnormals
    v[0, 4] = 1000.0 + (np.arange(H) % 7) * 0.001                                     # sums near 1000
    v[1:, 4] = rng.standard_normal((R - 1, H)) * 0.002
    v[:, 5] = rng.standard_normal((R, H)) * 4000.0                                    # large magnitudes
    v[:, 6] = np.where(np.arange(H) % 2 == 0, 1.0, -1.0) * rng.uniform(0, 3, size=(R, H))
    v[:, 7] = rng.standard_normal((R, H)) * 1e-6                                      # tiny
    bits = synth.operands_from_values(v, dtype)
    bits[:, 1, ::3] |= np.uint16(0x8000)                                              # -0 mixed with +0
    return bits


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_edge_groups(dtype, bits):
    x = _edge_values(dtype)
    w = synth.workload("tiny").with_(name="edge", R=4, T=8, H=512, bits=bits, group=128, dtype=dtype)
    ref = oracle.allreduce(x, dtype, bits, 128, want_f32=False)
    _say(f"edge groups {dtype} bits={bits}")
    _check(_run_fused(x, w), ref, w, x)          # the single launch (R*T*H <= 2^24)
    _check(_run_steps(x, w), ref, w, x)          # the three stage kernels


# ---------------------------------------------------------------------------
# determinism and agreement of the two ways in
# ---------------------------------------------------------------------------

def test_repeat_runs_and_entry_points_agree():
    w = synth.workload("llama3_8b_prefill").with_(T=1024)
    x = synth.operands(w, 3)
    _say("determinism: fused twice + separate entry points, 8B shape T=1024")
    a = _run_fused(x, w)
    b = _run_fused(x, w)
    c = _run_steps(x, w)
    for k in PAYLOAD + ("out",):
        assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


# ---------------------------------------------------------------------------
# different code widths before the reduce-scatter and the all-gather
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,bits2", [(4, 8), (8, 4)])
@pytest.mark.parametrize("name", ["llama3_70b_prefill", "llama3_8b_prefill", "decode", "sweep_int4_g4096"])
def test_mixed_widths(name, bits, bits2):
    w = synth.workload(name).with_(bits=bits)
    if w.T > 1024:
        w = w.with_(T=1024)
    x = synth.operands(w, 2)
    ref = oracle.allreduce(x, w.dtype, bits, w.group, want_f32=False, bits2=bits2)
    _say(f"mixed widths {name} T={w.T} bits {bits}->{bits2}")
    _check(_run_fused(x, w, bits2), ref, w, x)
    _check(_run_steps(x, w, bits2), ref, w, x)


@pytest.mark.parametrize("R,T,H,group", [(3, 7, 384, 128), (8, 9, 8192, 8192), (2, 33, 1024, 8),
                                         (5, 3, 640, 128), (6, 11, 3072, 512), (2, 5, 48, 8)])
def test_mixed_widths_ragged(R, T, H, group):
    for bits, bits2 in ((4, 8), (8, 4)):
        w = synth.workload("tiny").with_(R=R, T=T, H=H, bits=bits, group=group, dtype=synth.BF16,
                                         outlier_frac=0.01, outlier_scale=20.0)
        x = synth.operands(w, 5)
        ref = oracle.allreduce(x, w.dtype, bits, group, want_f32=False, bits2=bits2)
        _say(f"mixed widths ragged R={R} T={T} H={H} g={group} bits {bits}->{bits2}")
        _check(_run_fused(x, w, bits2), ref, w, x)

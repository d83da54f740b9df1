"""GPU parity of the single-launch emulated all-reduce (launch-bound shapes:
R <= 8, stage-1 group == stage-2 group <= 512, R*T*H <= 2^24), through the C ABI.

fc_allreduce_emulated, _mixed and _residual take this path for such shapes
and the three stage launches otherwise. Method: "Flash Communication: ..."
(Figure 5, right; Figure 3 for the residual add).

Bar: both payloads and the output bit-exact against the CPU oracle, for every
code width pair, both dtypes, with and without the residual add (also in
place); in addition the same bits as the three separate stage entry points on
the same device inputs; and both sides of the size threshold.
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
SMALL_MAX = 1 << 24   # R * T * H of the largest single-launch call


def _say(msg: str) -> None:
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


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


def _operands(R, T, H, dtype, seed):
    w = synth.workload("tiny").with_(name="small", R=R, T=T, H=H, bits=4, group=128, dtype=dtype,
                                     outlier_frac=0.01, outlier_scale=20.0)
    return synth.operands(w, seed)


def _fused(x, dtype, bits, bits2, group, residual=None, in_place=False):
    R, T, H = x.shape
    xd = _dev(x, dtype)
    res = None if residual is None else _dev(residual, dtype)
    out = res if in_place else None
    out, ws = fc.fc_allreduce_emulated(xd, bits, group, out=out, bits2=bits2, residual=res)
    views = fc.workspace_views(ws, R, T, H, bits, group, bits2=bits2)
    torch.cuda.synchronize()
    got = {k: _np(v) for k, v in views.items()}
    got["out"] = _np(out)
    return got


def _steps(x, dtype, bits, bits2, group, residual=None):
    R, T, H = x.shape
    xd = _dev(x, dtype)
    c1, s1, z1 = fc.fc_quantize_groups(xd, bits, group)
    c2, s2, z2 = fc.fc_dequant_sum_requant(c1, s1, z1, R, T, H, bits, group, bits2=bits2)
    g2 = fc.fc_stage2_group(R, H, group)
    if residual is None:
        out = fc.fc_dequantize(c2, s2, z2, T, H, bits2, g2, TDT[dtype])
    else:
        out = fc.fc_dequantize_residual(c2, s2, z2, T, H, bits2, g2, _dev(residual, dtype))
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in zip(PAYLOAD + ("out",), (c1, s1, z1, c2, s2, z2, out))}


def _oracle(x, dtype, bits, bits2, group, residual=None):
    R, T, H = x.shape
    ref = oracle.allreduce(x, dtype, bits, group, want_f32=False, bits2=bits2)
    if residual is not None:
        ref["out"] = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], T, H, bits2,
                                                ref["group2"], dtype, residual)
    return ref


def _same(got, want, what):
    for k in PAYLOAD + ("out",):
        a = np.asarray(got[k]).reshape(-1)
        b = np.asarray(want[k]).reshape(-1)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{what}: {k} differs at {bad.size} of {a.size}, first {bad[:6]}")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("bits,bits2", [(4, 4), (4, 8), (8, 4), (8, 8)])
@pytest.mark.parametrize("with_res", [False, True])
def test_every_variant_decode_shape(dtype, bits, bits2, with_res):
    """The decode shape (R = 8, T = 64, H = 8192, group 128): oracle and the
    three separate entry points."""
    R, T, H, group = 8, 64, 8192, 128
    _say(f"single launch decode {dtype} int{bits}->int{bits2} residual={with_res}")
    x = _operands(R, T, H, dtype, seed=11 + bits + bits2)
    res = None
    if with_res:
        rng = np.random.default_rng(5)
        v = rng.standard_normal((T, H)) * 2.0
        res = oracle.float_to_half(v) if dtype == synth.F16 else oracle.float_to_bf16(v)
    got = _fused(x, dtype, bits, bits2, group, res)
    _same(got, _oracle(x, dtype, bits, bits2, group, res), "vs oracle")
    _same(got, _steps(x, dtype, bits, bits2, group, res), "vs three launches")


@pytest.mark.parametrize("R,T,H,group", [
    (1, 3, 40, 8),        # one operand, 120 positions: the single slot ends early
    (2, 5, 64, 16),       # group 16, 320 positions: the slot ends early
    (3, 7, 384, 128),     # R = 3
    (5, 3, 640, 128),     # R = 5
    (7, 5, 7168, 512),    # the largest group of the path (a whole slot)
    (8, 33, 2048, 256),   # R = 8, group 256
    (4, 2, 4096, 32),     # group 32
])
def test_shapes(R, T, H, group):
    _say(f"single launch R={R} T={T} H={H} g={group}")
    for dtype, bits, bits2 in ((synth.BF16, 4, 4), (synth.F16, 8, 4)):
        x = _operands(R, T, H, dtype, seed=R * 100 + T)
        got = _fused(x, dtype, bits, bits2, group)
        _same(got, _oracle(x, dtype, bits, bits2, group), f"R={R} T={T} H={H} g={group}")


def test_residual_in_place():
    R, T, H, group = 4, 16, 1024, 128
    _say("single launch residual in place")
    x = _operands(R, T, H, synth.BF16, seed=3)
    rng = np.random.default_rng(9)
    res = oracle.float_to_bf16(rng.standard_normal((T, H)))
    got = _fused(x, synth.BF16, 4, 4, group, res, in_place=True)
    _same(got, _oracle(x, synth.BF16, 4, 4, group, res), "in place")


@pytest.mark.parametrize("T", [1024, 1025])
def test_threshold(T):
    """R*T*H = 2^24 takes the single launch, one token more the three launches:
    both bit-exact against the oracle."""
    R, H, group = 4, 4096, 128
    assert (R * T * H <= SMALL_MAX) == (T == 1024)
    _say(f"threshold R={R} T={T} H={H}")
    x = _operands(R, T, H, synth.BF16, seed=T)
    got = _fused(x, synth.BF16, 4, 4, group)
    _same(got, _oracle(x, synth.BF16, 4, 4, group), f"T={T}")


def test_stream_handle_is_torchs_current_stream():
    """The binding passes torch's current stream (raw handle) to the library,
    also inside a `torch.cuda.stream` context, and a call made there is ordered
    on that stream."""
    from bit_activation_compression_amd import _stream
    dev = torch.device("cuda", torch.cuda.current_device())
    assert _stream(None, dev).value == torch.cuda.current_stream(dev).cuda_stream or \
        (_stream(None, dev).value is None and torch.cuda.current_stream(dev).cuda_stream == 0)
    side = torch.cuda.Stream()
    x = _dev(_operands(2, 8, 256, synth.F16, seed=1), synth.F16)
    ref, _ = fc.fc_allreduce_emulated(x, 8, 128)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        assert _stream(None, dev).value == side.cuda_stream
        out, _ = fc.fc_allreduce_emulated(x, 8, 128)
    side.synchronize()
    assert torch.equal(out, ref)

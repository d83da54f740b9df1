"""GPU parity of the final dequantize fused with the residual add (Figure 3 of
"Flash Communication: ...": the all-reduced attention and MLP outputs are added
to the residual stream), through the C ABI against the CPU oracle.

Bar: bit-exact. out = round(residual + round(q*s + z)) takes the same two
roundings on both sides. Payloads and residuals come from the seeded generator
and the oracle, never from the GPU.
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


def _say(msg: str) -> None:
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    fc.lib()
    yield


def _to_dev(a: np.ndarray, torch_dtype=None) -> torch.Tensor:
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).cuda()
        return t.view(torch_dtype) if torch_dtype is not None else t.view(torch.uint16)
    return torch.from_numpy(a).cuda()


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _residual(w: synth.Workload, seed: int, T: int | None = None) -> np.ndarray:
    """The residual stream: one more seeded activation of shape [T, H]."""
    tok = None if T is None else slice(0, T)
    return synth.operands(w.with_(R=1, sigma=4.0 * w.sigma), seed + 7919, tokens=tok)[0]


CASES = [
    ("tiny", 0), ("decode", 0), ("llama3_8b_prefill", 0),
]


@pytest.mark.parametrize("name,seed", CASES)
def test_dequantize_residual_matches_oracle(name, seed):
    w = synth.workload(name)
    T = min(w.T, 512)          # the oracle's share; several tiles and a full row set
    x = synth.operands(w, seed, tokens=slice(0, T))
    _say(f"dequantize_residual {name} seed={seed} T={T}")
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    res = _residual(w, seed, T)
    expect = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], T, w.H, w.bits,
                                        ref["group2"], w.dtype, res)
    c2, s2, z2 = (_to_dev(ref[k]) for k in ("codes2", "s2", "z2"))
    rd = _to_dev(res, TDT[w.dtype])
    out = fc.fc_dequantize_residual(c2, s2, z2, T, w.H, w.bits, ref["group2"], rd)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), expect)
    # in place: the residual stream updated where it lies
    fc.fc_dequantize_residual(c2, s2, z2, T, w.H, w.bits, ref["group2"], rd, out=rd)
    torch.cuda.synchronize()
    assert np.array_equal(_np(rd), expect)


@pytest.mark.parametrize("bits,bits2", [(4, 4), (8, 8), (4, 8)])
@pytest.mark.parametrize("name", ["llama3_70b_prefill", "decode", "sweep_int8_g4096"])
def test_allreduce_with_residual_matches_oracle(name, bits, bits2):
    w = synth.workload(name).with_(bits=bits)
    T = min(w.T, 256)
    x = synth.operands(w, 3, tokens=slice(0, T))
    _say(f"allreduce_emulated_residual {name} int{bits}->int{bits2} T={T}")
    ref = oracle.allreduce(x, w.dtype, bits, w.group, want_f32=False, bits2=bits2)
    res = _residual(w, 3, T)
    expect = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], T, w.H, bits2,
                                        ref["group2"], w.dtype, res)
    xd = _to_dev(x, TDT[w.dtype])
    rd = _to_dev(res, TDT[w.dtype])
    out, ws = fc.fc_allreduce_emulated(xd, bits, w.group, bits2=bits2, residual=rd)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), expect)
    views = fc.workspace_views(ws, w.R, T, w.H, bits, w.group, bits2=bits2)
    for k in ("codes1", "s1", "z1", "codes2", "s2", "z2"):
        assert np.array_equal(_np(views[k]).reshape(-1), ref[k].reshape(-1)), k


RAGGED = [  # (T, H, bits, group2, dtype): T*H not a multiple of a wave's 2048 elements
    (1, 8, 8, 8, synth.F16),
    (5, 40, 4, 8, synth.BF16),
    (3, 1000, 8, 8, synth.F16),
    (7, 8192, 4, 8192, synth.BF16),
    (33, 1024, 4, 128, synth.F16),
]


@pytest.mark.parametrize("T,H,bits,group2,dtype", RAGGED)
def test_ragged_shapes(T, H, bits, group2, dtype):
    _say(f"dequantize_residual ragged T={T} H={H} int{bits} g{group2} {dtype}")
    w = synth.Workload("ragged", R=1, T=T, H=H, dtype=dtype, bits=bits, group=group2)
    v = synth.operands(w, 11)[0]
    # a stage-2 payload from the oracle's quantizer on binary32 values
    widen = oracle.half_to_float if dtype == synth.F16 else oracle.bf16_to_float
    codes, s, z = oracle.quantize_f32(widen(v).reshape(-1), bits, group2)
    codes = codes.reshape(T, H * bits // 8)
    s, z = s.reshape(T, H // group2), z.reshape(T, H // group2)
    res = _residual(w, 11)
    expect = oracle.dequantize_residual(codes, s, z, T, H, bits, group2, dtype, res)
    out = fc.fc_dequantize_residual(_to_dev(codes), _to_dev(s), _to_dev(z), T, H, bits, group2,
                                    _to_dev(res, TDT[dtype]))
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), expect)


def test_empty_token_dimension():
    _say("dequantize_residual T=0")
    e8 = torch.empty(0, dtype=torch.uint8, device="cuda")
    e16 = torch.empty(0, dtype=torch.uint16, device="cuda")
    res = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = fc.fc_dequantize_residual(e8, e16, e16, 0, 256, 4, 128, res)
    assert out.shape == (0, 256)


def test_full_size_sampled_rows():
    """LLaMA-3-70B prefill at full size (R=4, T=8192, H=8192, bf16, INT4, g=128)
    in the launch the benchmark times; rows sampled across the whole range are
    recomputed by the oracle from the same seeded operands (each output row
    depends only on the same row of the R operands)."""
    w = synth.workload("llama3_70b_prefill")
    _say("allreduce_emulated_residual llama3_70b_prefill full size")
    x = synth.operands(w, 0)
    res = _residual(w, 0)
    xd = _to_dev(x, TDT[w.dtype])
    rd = _to_dev(res, TDT[w.dtype])
    out, _ = fc.fc_allreduce_emulated(xd, w.bits, w.group, residual=rd)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 17, 1023, 4096, 5555, w.T - 2, w.T - 1])
    got = _np(out[torch.from_numpy(rows).cuda()])
    ref = oracle.allreduce(np.ascontiguousarray(x[:, rows]), w.dtype, w.bits, w.group,
                           want_f32=False)
    expect = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], len(rows), w.H,
                                        w.bits, ref["group2"], w.dtype,
                                        np.ascontiguousarray(res[rows]))
    assert np.array_equal(got, expect)

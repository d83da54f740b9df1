"""GPU parity of the uncompressed all-reduce comparator (fc_sum_uncompressed)
against the CPU oracle: bit-exact on full workloads, ragged shapes and edge
values. Comparator of "Flash Communication: ..." Figure 1 (ring all-reduce of
FP16 activations)."""
import sys

import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle
import synth

pytestmark = pytest.mark.gpu
TDT = {synth.F16: torch.float16, synth.BF16: torch.bfloat16}


def _say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _run(x: np.ndarray, dtype: str) -> np.ndarray:
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(TDT[dtype])
    out = fc.fc_sum_uncompressed(xd)
    torch.cuda.synchronize()
    return out.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "llama3_8b_prefill", "llama3_70b_prefill", "decode"])
def test_full_workloads(name):
    w = synth.workload(name)
    x = synth.operands(w, 0)
    _say(f"uncompressed sum {name}")
    assert np.array_equal(_run(x, w.dtype), oracle.sum_uncompressed(x, w.dtype))


@pytest.mark.parametrize("R,T,H,dtype", [(1, 3, 8, synth.F16), (3, 7, 24, synth.BF16),
                                         (5, 33, 1000, synth.F16), (8, 2, 4104, synth.BF16),
                                         (6, 129, 520, synth.F16)])
def test_ragged(R, T, H, dtype):
    w = synth.workload("tiny").with_(R=R, T=T, H=H, dtype=dtype)
    x = synth.operands(w, 3)
    _say(f"uncompressed sum ragged R={R} T={T} H={H} {dtype}")
    assert np.array_equal(_run(x, dtype), oracle.sum_uncompressed(x, dtype))


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_edge_values(dtype):
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal((4, 2, 512)) * 1e-6, rng.standard_normal((4, 2, 512)) * 8000,
                        np.zeros((4, 1, 512))], axis=1)
    x = synth.operands_from_values(v, dtype)
    x[:, 4, ::2] |= np.uint16(0x8000)          # -0 operands
    _say(f"uncompressed sum edge values {dtype}")
    assert np.array_equal(_run(x, dtype), oracle.sum_uncompressed(x, dtype))


def test_empty():
    x = torch.empty((4, 0, 64), dtype=torch.float16, device="cuda")
    out = fc.fc_sum_uncompressed(x)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)

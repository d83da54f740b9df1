"""The C oracle against the independent numpy re-derivation (tests/np_ref.py),
bit for bit on every intermediate, at reduced token counts of every workload.
This is a consistency check of two statements of the same reading of the
Flash Communication page (Figure 4; Figure 5, right), not a pin on its own."""
import numpy as np
import pytest

import oracle
import synth
from np_ref import allreduce as np_allreduce

CASES = ["tiny", "llama3_8b_prefill", "llama3_70b_prefill", "decode"] + [
    f"sweep_int{b}_g{g}" for b in synth.SWEEP_BITS for g in synth.SWEEP_GROUPS]


@pytest.mark.parametrize("name", CASES)
def test_c_oracle_equals_numpy_rederivation(name):
    w = synth.workload(name)
    w = w.with_(T=min(w.T, 24))
    for seed in (0, 1):
        x = synth.operands(w, seed)
        a = oracle.allreduce(x, w.dtype, w.bits, w.group)
        b = np_allreduce(x, w.dtype, w.bits, w.group)
        for k in ("codes1", "s1", "z1", "codes2", "s2", "z2", "out"):
            assert np.array_equal(a[k].reshape(-1), b[k].reshape(-1)), (name, seed, k)
        assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))
        assert np.array_equal(a["o32"].view(np.uint32), b["o32"].view(np.uint32))


@pytest.mark.parametrize("R,H,g", [(1, 64, 64), (3, 96, 32), (2, 512, 256), (8, 256, 64)])
def test_odd_shapes(R, H, g):
    w = synth.workload("tiny").with_(R=R, H=H, group=g, T=5, bits=4)
    x = synth.operands(w, 4)
    a = oracle.allreduce(x, w.dtype, w.bits, w.group)
    b = np_allreduce(x, w.dtype, w.bits, w.group)
    for k in ("codes1", "s1", "z1", "codes2", "s2", "z2", "out"):
        assert np.array_equal(a[k].reshape(-1), b[k].reshape(-1)), k


@pytest.mark.parametrize("bits,bits2", [(4, 8), (8, 4)])
@pytest.mark.parametrize("name", ["llama3_8b_prefill", "llama3_70b_prefill", "decode", "sweep_int4_g4096"])
def test_mixed_widths_equal_numpy_rederivation(name, bits, bits2):
    w = synth.workload(name)
    w = w.with_(T=min(w.T, 16))
    x = synth.operands(w, 6)
    a = oracle.allreduce(x, w.dtype, bits, w.group, bits2=bits2)
    b = np_allreduce(x, w.dtype, bits, w.group, bits2=bits2)
    for k in ("codes1", "s1", "z1", "codes2", "s2", "z2", "out"):
        assert np.array_equal(a[k].reshape(-1), b[k].reshape(-1)), (name, k)

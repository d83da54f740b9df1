"""fc_allreduce_emulated_noalloc through the C ABI on the GPU: the output equals
fc_allreduce_emulated's (caller workspace) bit for bit, on consecutive calls that
share the library's scratch, each smaller than the one before; the largest shape
that fits the scratch runs and the next larger one is rejected with nothing
written. Inputs: the seeded synthetic generator."""
import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _x(w, seed):
    x = synth.operands(w, seed)
    tdt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float16
    return x, torch.from_numpy(x.view(np.int16)).to(DEV).view(tdt)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# three-launch path (R*T*H > 2^24), then the single launch (decode), then a tiny one
CASES = [
    ("llama3_8b_prefill", dict(T=1100)),
    ("decode", dict()),
    ("tiny", dict()),
]


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls():
    stream = torch.cuda.current_stream(DEV)
    for rep in range(2):
        for i, (name, kw) in enumerate(CASES):
            w = synth.workload(name).with_(**kw)
            print(f"[noalloc] rep {rep} call {i}: {name} R={w.R} T={w.T} H={w.H} int{w.bits} "
                  f"g{w.group} {w.dtype}", flush=True)
            assert fc.fc_workspace_bytes(w.R, w.T, w.H, w.bits, w.group) <= fc.NOALLOC_SCRATCH_BYTES
            _, xd = _x(w, 7 + i + rep)
            ref, _ = fc.fc_allreduce_emulated(xd, w.bits, w.group, stream=stream)
            out = torch.empty_like(ref).fill_(7.0)
            fc.fc_allreduce_emulated_noalloc(xd, w.bits, w.group, out, stream=stream)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(out), _bits(ref)), (name, rep)


def test_noalloc_matches_oracle_tiny():
    w = synth.workload("tiny")
    x, xd = _x(w, 3)
    out = torch.empty((w.T, w.H), dtype=xd.dtype, device=DEV)
    fc.fc_allreduce_emulated_noalloc(xd, w.bits, w.group, out)
    torch.cuda.synchronize()
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False)
    assert np.array_equal(_bits(out), ref["out"])


def test_noalloc_largest_shape_fits_and_next_is_rejected():
    R, H, bits, g = 4, 8192, 4, 128
    T = 1
    while fc.fc_workspace_bytes(R, 2 * T, H, bits, g) <= fc.NOALLOC_SCRATCH_BYTES:
        T *= 2
    lo, hi = T, 2 * T
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if fc.fc_workspace_bytes(R, mid, H, bits, g) <= fc.NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid
    print(f"[noalloc] largest T = {lo} for R={R} H={H} int{bits} g{g}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(1)
    xd = (torch.randn((R, lo, H), generator=gen, device=DEV) * 0.5).to(torch.bfloat16)
    ref, _ = fc.fc_allreduce_emulated(xd, bits, g)
    out = torch.empty_like(ref)
    fc.fc_allreduce_emulated_noalloc(xd, bits, g, out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))
    big = torch.zeros((R, lo + 1, H), dtype=xd.dtype, device=DEV)
    out2 = torch.full((lo + 1, H), 3.0, dtype=xd.dtype, device=DEV)
    with pytest.raises(fc.FcError) as e:
        fc.fc_allreduce_emulated_noalloc(big, bits, g, out2)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((out2 == 3.0).all())


@pytest.mark.parametrize("name,kw", [("decode", {}), ("llama3_8b_prefill", {"T": 1100})])
def test_noalloc_captured_in_a_graph(name, kw):
    """The callers this entry point is for capture it in HIP graphs: every replay reproduces
    the eager result, also after an eager call of another shape has overwritten the shared
    scratch in between (each call writes its payloads before it reads them)."""
    w = synth.workload(name).with_(**kw)
    print(f"[noalloc] graph capture {name} R={w.R} T={w.T} H={w.H}", flush=True)
    _, xd = _x(w, 5)
    ref, _ = fc.fc_allreduce_emulated(xd, w.bits, w.group)
    torch.cuda.synchronize()
    want = _bits(ref)
    out = torch.empty_like(ref)
    other_w = synth.workload("tiny")
    _, xo = _x(other_w, 6)
    out_o = torch.empty((other_w.T, other_w.H), dtype=xo.dtype, device=DEV)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fc.fc_allreduce_emulated_noalloc(xd, w.bits, w.group, out, stream=cap)
        with torch.cuda.graph(graph, stream=cap):
            fc.fc_allreduce_emulated_noalloc(xd, w.bits, w.group, out, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        fc.fc_allreduce_emulated_noalloc(xo, other_w.bits, other_w.group, out_o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), want), f"replay {i}"

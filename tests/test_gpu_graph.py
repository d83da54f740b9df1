"""The codec captured in a HIP graph and replayed: every replay, with eager
work and synchronizations in between, must reproduce the eager result bit
for bit (the decode shape of "Flash Communication: ...", where launches
dominate the latency)."""
import sys

import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits2", [None, 8])
def test_graph_replays_match_eager_and_oracle(bits2):
    w = synth.workload("decode")
    print(f"[gpu] graph capture decode bits2={bits2}", file=sys.stderr, flush=True)
    x = synth.operands(w, 0)
    ref = oracle.allreduce(x, w.dtype, w.bits, w.group, want_f32=False, bits2=bits2)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    out, ws = fc.fc_allreduce_emulated(xd, w.bits, w.group, bits2=bits2)
    torch.cuda.synchronize()
    eager = out.clone()
    assert np.array_equal(eager.cpu().view(torch.int16).numpy().view(np.uint16), ref["out"])
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            fc.fc_allreduce_emulated(xd, w.bits, w.group, out, ws, stream=cap, bits2=bits2)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"

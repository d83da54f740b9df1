"""Beyond 2^32 values: R=4 operands of T=139264 x H=8192 bf16 (4.6e9 values,
9.1 GB). Every kernel indexes tiles with 64-bit offsets; this checks that the
payloads and output of token rows on both sides of the 2^32-element mark (and
the first and last rows) match the CPU oracle bit for bit. The input is drawn
on the GPU by torch's seeded generator (not the codec) and the sampled rows
are copied back for the oracle, which processes only those rows."""
import sys

import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle

pytestmark = pytest.mark.gpu


def test_beyond_2_pow_32_values():
    R, T, H, bits, g = 4, 139264, 8192, 4, 128
    assert R * T * H > 2 ** 32
    free, _ = torch.cuda.mem_get_info()
    if free < 20 * 2 ** 30:
        pytest.skip("needs ~14 GB of free device memory")
    print(f"[gpu] large: R={R} T={T} H={H} ({R * T * H} values)", file=sys.stderr, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    x = torch.empty((R, T, H), dtype=torch.bfloat16, device="cuda")
    for r in range(R):
        x[r] = (torch.randn((T, H), generator=gen, device="cuda", dtype=torch.float32) * 0.5).to(torch.bfloat16)
    out, ws = fc.fc_allreduce_emulated(x, bits, g)
    v = fc.workspace_views(ws, R, T, H, bits, g)
    torch.cuda.synchronize()
    # rows: first, last, around operand r's crossing of element 2^32 (operand 2 starts at 2*T*H)
    cross = (2 ** 32) // H
    rows = sorted({0, T - 1, 1, cross % T, (cross + 1) % T, T // 2, T // 2 + 1, T - 2})
    xs = x[:, rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.allreduce(xs, oracle.BF16, bits, g, want_f32=False)
    def rows_of(t, operand_axis):   # 16-bit tensors are indexed through an int16 view
        t = t.view(torch.int16) if t.element_size() == 2 else t
        t = t[:, rows] if operand_axis else t[rows]
        a = t.contiguous().cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a
    assert np.array_equal(rows_of(v["codes1"], True), ref["codes1"])
    assert np.array_equal(rows_of(v["s1"], True), ref["s1"])
    assert np.array_equal(rows_of(v["z1"], True), ref["z1"])
    assert np.array_equal(rows_of(v["codes2"], False), ref["codes2"])
    assert np.array_equal(rows_of(v["s2"], False), ref["s2"])
    assert np.array_equal(rows_of(v["z2"], False), ref["z2"])
    assert np.array_equal(rows_of(out, False), ref["out"])
    # the uncompressed comparator on the same rows
    sref = oracle.sum_uncompressed(xs, oracle.BF16)
    s = fc.fc_sum_uncompressed(x)
    torch.cuda.synchronize()
    assert np.array_equal(rows_of(s, False), sref)


@pytest.mark.parametrize("H,g", [(8192, 128), (6144, 96)])
def test_beyond_2_pow_32_output_positions(H, g):
    """T*H past 2^32 (R=2 operands of fp16, ~17 GB): the reduction and the
    final dequantize index output positions and their groups in 64 bits (the
    generic kernels divide by the group length in 64 bits there). Rows on
    both sides of position 2^32, the first and the last, against the oracle."""
    R, bits = 2, 4
    T = (2 ** 32) // H + 6
    assert T * H > 2 ** 32
    free, _ = torch.cuda.mem_get_info()
    need = R * T * H * 2 + R * T * H // 2 + T * H * 2 + T * H
    if free < need + 8 * 2 ** 30:
        pytest.skip(f"needs ~{need / 2 ** 30:.0f} GB of free device memory")
    print(f"[gpu] large: R={R} T={T} H={H} g={g} ({T * H} output positions)", file=sys.stderr, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(99)
    x = torch.empty((R, T, H), dtype=torch.float16, device="cuda")
    step = 65536
    for r in range(R):
        for t0 in range(0, T, step):
            t1 = min(T, t0 + step)
            x[r, t0:t1] = torch.randn((t1 - t0, H), generator=gen, device="cuda",
                                      dtype=torch.float32).to(torch.float16)
    out, ws = fc.fc_allreduce_emulated(x, bits, g)
    v = fc.workspace_views(ws, R, T, H, bits, g)
    torch.cuda.synchronize()
    cross = (2 ** 32) // H
    rows = sorted({0, 1, cross - 1, cross, cross + 1, T - 2, T - 1})
    xs = x[:, rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.allreduce(xs, oracle.F16, bits, g, want_f32=False)

    def rows_of(t, operand_axis):
        t = t.view(torch.int16) if t.element_size() == 2 else t
        t = t[:, rows] if operand_axis else t[rows]
        a = t.contiguous().cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(rows_of(v[k], True), ref[k]), k
    for k in ("codes2", "s2", "z2"):
        assert np.array_equal(rows_of(v[k], False), ref[k]), k
    assert np.array_equal(rows_of(out, False), ref["out"])
    del x, out, ws, v
    torch.cuda.empty_cache()

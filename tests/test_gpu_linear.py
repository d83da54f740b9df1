"""GPU parity of the row-parallel linear layer with the stage-1 quantization in
its epilogue (Figure 3 of "Flash Communication: ...": o_proj / d_proj end in
the all-reduce), through the C ABI against the CPU oracle.

Bar:
  - dyadic inputs (small integers times powers of two): every product and
    partial sum is exact in binary32, so the layer output is unique whatever
    the accumulation order -- y, codes, scales and zeros bit-exact;
  - normal inputs: y within the binary32 accumulation bound of the oracle's
    y; codes bit-exact on every group whose y matches the oracle's exactly
    (the codes are a function of y), and equal to fc_quantize_groups applied
    to this call's own y everywhere.
Inputs are seeded on the host; nothing the oracle sees comes from the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import bit_activation_compression_amd as fc
import oracle

pytestmark = pytest.mark.gpu

TDT = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}


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
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _bits(v: np.ndarray, dtype: str) -> np.ndarray:
    v32 = np.asarray(v, dtype=np.float32)
    if dtype == oracle.F16:
        return oracle.float_to_half(v32)
    return oracle.float_to_bf16(v32)


def _dyadic(rng, R, T, K, H, dtype):
    """a = ka/8, w = kw/64 with |ka|, |kw| <= 8 and a few output channels x16:
    |sum| <= K * 8 * 8 * 16 units of 2^-9 < 2^24 for K < 16384 -- exact."""
    ka = rng.integers(-8, 9, size=(R, T, K), dtype=np.int8).astype(np.float32) / 8
    kw = rng.integers(-8, 9, size=(R, H, K), dtype=np.int8).astype(np.float32) / 64
    hot = rng.choice(H, size=max(1, H // 100), replace=False)
    kw[:, hot] *= 16
    return _bits(ka, dtype), _bits(kw, dtype)


def _run(a, w, dtype, bits, group, want_y=True):
    ad, wd = _dev(a, dtype), _dev(w, dtype)
    c, s, z, y = fc.fc_linear_quantize(ad, wd, bits, group, y=True if want_y else None)
    torch.cuda.synchronize()
    return {"codes1": _np(c), "s1": _np(s), "z1": _np(z), "y": _np(y) if want_y else None}


EXACT = [  # (R, T, K, H, group, bits, dtype)
    (1, 256, 32, 256, 128, 4, oracle.BF16),     # one tile, a single k stage
    (1, 256, 64, 256, 128, 4, oracle.BF16),     # two stages
    (2, 260, 96, 256, 64, 4, oracle.F16),       # three stages, ragged tokens
    (2, 100, 128, 512, 128, 8, oracle.BF16),    # four stages: the ring turns over once
    (2, 260, 320, 256, 64, 4, oracle.F16),      # ten stages
    (2, 300, 128, 512, 64, 8, oracle.F16),      # ragged tokens
    (4, 37, 192, 1024, 32, 4, oracle.BF16),     # fewer tokens than a tile, 6 stages
    (4, 520, 256, 768, 8, 8, oracle.BF16),      # group 8; 36 tiles (no XCD regrouping)
    (3, 256, 64, 768, 16, 4, oracle.F16),       # R = 3
    (4, 512, 2048, 8192, 128, 4, oracle.BF16),  # LLaMA-3-70B o_proj per rank, 512 tokens
    (2, 64, 1024, 4096, 128, 8, oracle.F16),    # decode-sized token count
    (2, 2000, 3072, 512, 64, 8, oracle.F16),    # XCD-grid tile order (K >= 3072), ragged tokens
    (1, 1000, 3200, 512, 32, 4, oracle.BF16),   # XCD grid with one tile per XCD
    (2, 2048, 3136, 1024, 16, 4, oracle.F16),   # XCD grid, 2 x 2 tiles per XCD and rank
    (3, 1024, 3104, 768, 128, 8, oracle.F16),   # K >= 3072 but 3 channel tiles: XCD runs; odd stage count
    (2, 300, 352, 512, 8, 4, oracle.F16),       # 4-bit codes in groups of 8 (staging loads in one burst), 11 stages
    (1, 700, 160, 256, 8, 4, oracle.BF16),      # the same, bf16, 5 stages
    (2, 300, 160, 512, 256, 4, oracle.BF16),    # groups of 256: a tile row, split over two waves
    (1, 257, 64, 256, 256, 8, oracle.F16),      # the same, one channel tile, INT8
    (2, 2048, 3072, 512, 256, 4, oracle.F16),   # the same on the XCD grid
    # long rows (K >= 3072) also prefetch into L2
    (1, 300, 3104, 256, 8, 4, oracle.BF16),     # 4-bit codes in groups of 8, odd stage count
    (2, 1792, 3072, 512, 128, 4, oracle.F16),   # 7 token tiles: scheduling groups of 4 and 3
    (1, 512, 3072, 512, 16, 8, oracle.BF16),    # INT8 in groups of 16 (the largest LDS use)
]


@pytest.mark.parametrize("R,T,K,H,group,bits,dtype", EXACT)
def test_dyadic_inputs_bit_exact(R, T, K, H, group, bits, dtype):
    _say(f"linear_quantize dyadic R={R} T={T} K={K} H={H} g{group} int{bits} {dtype}")
    rng = np.random.default_rng(1000 + R * T + K + H + group + bits)
    a, w = _dyadic(rng, R, T, K, H, dtype)
    ref = oracle.linear_quantize(a, w, dtype, bits, group)
    got = _run(a, w, dtype, bits, group)
    assert np.array_equal(got["y"], ref["y"])
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got[k], ref[k]), k
    # without the y output: the same codes
    got2 = _run(a, w, dtype, bits, group, want_y=False)
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got2[k], ref[k]), k


def _draw_linear(rng):
    """A supported (R, T, K, H, group, bits, dtype): K a multiple of 32 (odd
    stage counts included: the last staged pair is then half used), H a
    multiple of 256 and of R, group <= 256; sizes kept small."""
    R = int(rng.integers(1, 5))
    K = 32 * int(rng.integers(1, 24))
    H = 256 * int(rng.integers(1, 5))
    if H % R:
        H *= R                                   # H % R == 0 (the chunking needs it)
    T = int(rng.integers(1, 600))
    group = int(2 ** rng.integers(3, 9))
    bits = int(rng.choice([4, 8]))
    dtype = oracle.F16 if rng.random() < 0.5 else oracle.BF16
    return R, T, K, H, group, bits, dtype


RANDOM = [_draw_linear(np.random.default_rng(77 + i)) for i in range(32)]


@pytest.mark.parametrize("R,T,K,H,group,bits,dtype", RANDOM)
def test_random_dyadic_shapes(R, T, K, H, group, bits, dtype):
    _say(f"linear_quantize random R={R} T={T} K={K} H={H} g{group} int{bits} {dtype}")
    rng = np.random.default_rng(R * T + K * 3 + H)
    a, w = _dyadic(rng, R, T, K, H, dtype)
    ref = oracle.linear_quantize(a, w, dtype, bits, group)
    got = _run(a, w, dtype, bits, group)
    assert np.array_equal(got["y"], ref["y"])
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got[k], ref[k]), k


def _ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the dtype at |v| (normal range)."""
    p = 11 if dtype == oracle.F16 else 8
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    return 2.0 ** (e - p + 1)


@pytest.mark.parametrize("R,T,K,H,group,bits,dtype", [
    (4, 256, 2048, 8192, 128, 4, oracle.BF16),
    (2, 200, 512, 1024, 32, 8, oracle.F16),
])
def test_normal_inputs(R, T, K, H, group, bits, dtype):
    _say(f"linear_quantize normal R={R} T={T} K={K} H={H} g{group} int{bits} {dtype}")
    rng = np.random.default_rng(77 + K)
    a = _bits(rng.normal(size=(R, T, K)), dtype)
    w = _bits(rng.normal(size=(R, H, K)) / np.sqrt(K), dtype)
    ref = oracle.linear_quantize(a, w, dtype, bits, group)
    got = _run(a, w, dtype, bits, group)
    widen = oracle.half_to_float if dtype == oracle.F16 else oracle.bf16_to_float
    yg = widen(got["y"]).astype(np.float64)
    yr = widen(ref["y"]).astype(np.float64)
    # binary32 accumulation of K exact products in any order: |err| <= 2K u sum|a w|
    absdot = np.matmul(np.abs(widen(a).astype(np.float64)),
                       np.abs(widen(w).astype(np.float64)).transpose(0, 2, 1))
    bound = _ulp(np.maximum(np.abs(yg), np.abs(yr)), dtype) + 2 * K * 2.0 ** -24 * absdot
    assert np.all(np.abs(yg - yr) <= bound)
    # groups whose stored y equals the oracle's: codes, scales, zeros identical
    same = (got["y"] == ref["y"]).reshape(R, T, H // group, group).all(-1)
    assert same.mean() > 0.5
    s_ok = got["s1"][same] == ref["s1"][same]
    z_ok = got["z1"][same] == ref["z1"][same]
    assert s_ok.all() and z_ok.all()
    cg = got["codes1"].reshape(R, T, H // group, group * bits // 8)
    cr = ref["codes1"].reshape(R, T, H // group, group * bits // 8)
    assert np.array_equal(cg[same], cr[same])
    # everywhere: the epilogue equals the stage-1 quantizer on this call's own y
    c2, s2, z2 = fc.fc_quantize_groups(_dev(got["y"], dtype), bits, group)
    torch.cuda.synchronize()
    assert np.array_equal(_np(c2), got["codes1"])
    assert np.array_equal(_np(s2), got["s1"]) and np.array_equal(_np(z2), got["z1"])


@pytest.mark.parametrize("bits,dtype", [(4, oracle.BF16), (8, oracle.F16)])
def test_degenerate_groups(bits, dtype):
    """Output groups whose values are all equal: zero weight rows give groups
    of zeros (scale 0), equal weight rows give constant nonzero groups, and
    a zero token row gives a whole row of zeros."""
    R, T, K, H, group = 2, 300, 96, 512, 128
    _say(f"linear_quantize degenerate groups int{bits} {dtype}")
    rng = np.random.default_rng(31)
    a, w = _dyadic(rng, R, T, K, H, dtype)
    w[:, 0:128] = _bits(np.zeros((R, 128, K), dtype=np.float32), dtype)          # y = 0
    w[:, 128:256] = w[:, 128:129]                                                  # equal channels
    a[:, 7] = _bits(np.zeros((R, K), dtype=np.float32), dtype)                    # a zero token row
    ref = oracle.linear_quantize(a, w, dtype, bits, group)
    got = _run(a, w, dtype, bits, group)
    assert np.array_equal(got["y"], ref["y"])
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.all(ref["s1"][:, :, 0] == 0) and np.all(ref["s1"][:, :, 1] == 0)   # the cases are hit


def test_empty_token_dimension():
    _say("linear_quantize T=0")
    a = torch.empty((4, 0, 2048), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, 8192, 2048), dtype=torch.bfloat16, device="cuda")
    c, s, z, _ = fc.fc_linear_quantize(a, w, 4, 128)
    assert c.shape == (4, 0, 4096) and s.shape == (4, 0, 64)


def test_full_size_sampled_rows():
    """LLaMA-3-70B attention output projection at full size, one GPU's share of
    TP = 4 (R=4, T=8192, K=2048, H=8192, bf16, INT4, g=128), the launch the
    benchmark times: dyadic inputs make every row's result unique, and rows
    sampled across the token range are recomputed by the oracle from the same
    host inputs."""
    R, T, K, H, group, bits, dtype = 4, 8192, 2048, 8192, 128, 4, oracle.BF16
    _say("linear_quantize full size 70B o_proj")
    rng = np.random.default_rng(4242)
    a, w = _dyadic(rng, R, T, K, H, dtype)
    got = _run(a, w, dtype, bits, group, want_y=False)
    rows = np.array([0, 1, 255, 256, 4097, 6000, T - 2, T - 1])
    ref = oracle.linear_quantize(np.ascontiguousarray(a[:, rows]), w, dtype, bits, group)
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got[k][:, rows], ref[k]), k


def test_full_size_d_proj_sampled_rows():
    """LLaMA-3-70B MLP down projection at full size, one GPU's share of TP = 4
    (R=4, T=8192, K=28672/4=7168, H=8192, bf16, INT4, g=128): the long-row
    launch, which takes its tiles on the XCD grid. Dyadic inputs (exact for
    K < 16384); sampled rows recomputed by the oracle."""
    R, T, K, H, group, bits, dtype = 4, 8192, 7168, 8192, 128, 4, oracle.BF16
    _say("linear_quantize full size 70B d_proj")
    rng = np.random.default_rng(4343)
    a, w = _dyadic(rng, R, T, K, H, dtype)
    got = _run(a, w, dtype, bits, group, want_y=False)
    rows = np.array([0, 255, 256, 2047, 2048, 5000, T - 1])
    ref = oracle.linear_quantize(np.ascontiguousarray(a[:, rows]), w, dtype, bits, group)
    for k in ("codes1", "s1", "z1"):
        assert np.array_equal(got[k][:, rows], ref[k]), k

"""Pins of the CPU oracle to things other than itself.

Method: "Flash Communication: Reducing Tensor Parallelization Bottleneck for
Fast Large Language Model Inference" -- TL;DR and Abstract (low-bit
activation codes around a two-step all-reduce), Figure 4 (block-wise groups
along the hidden dimension, from the hidden length down to 128), Figure 5,
right (quantization before the Reduce-Scatter and before the All-Gather).

Each test names what fixes its expected values: a library routine, a closed
form, a hand-derived fixture under tests/golden/, brute force over every
candidate code, or a bound that follows from the arithmetic.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16(vals) -> np.ndarray:
    a = np.asarray(vals, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.all(h.astype(np.float64) == a), "fixture value not exact in fp16"
    return h.view(np.uint16)


def _hval(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _unpack(codes: np.ndarray, bits: int) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.copy()
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


def _read_fixture(name: str) -> dict:
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            d[k] = v
    return d


# ---------------------------------------------------------------------------
# conversions, pinned to library routines (numpy float16, torch bfloat16)
# ---------------------------------------------------------------------------

def test_half_to_float_all_patterns_match_numpy():
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.half_to_float(h)
    ref = h.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def _f32_probe_values() -> np.ndarray:
    rng = np.random.default_rng(1234)
    h = np.arange(0, 0x7C00, dtype=np.uint16)              # every finite positive fp16
    f = h.view(np.float16).astype(np.float32)
    u = f.view(np.uint32).astype(np.int64)
    nb = [u, u + 1, u - 1]
    fh = f.astype(np.float64)
    mids = ((fh[:-1] + fh[1:]) / 2).astype(np.float32)   # exact midpoints (fit in fp32)
    mu = mids.view(np.uint32).astype(np.int64)
    nb += [mu, mu + 1, mu - 1]
    rnd = rng.integers(0, 0x7F800000, size=200000, dtype=np.int64)
    allu = np.concatenate(nb + [rnd, np.array([0x7F800000, 0x477FF000, 0x477FEFFF, 0x477FE000])])
    allu = allu[(allu >= 0) & (allu <= 0x7F800000)]
    pos = allu.astype(np.uint32).view(np.float32)
    return np.concatenate([pos, -pos])


def test_float_to_half_matches_numpy_rne():
    v = _f32_probe_values()
    got = oracle.float_to_half(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_conversions_match_torch():
    v = _f32_probe_values()
    rng = np.random.default_rng(7)
    small = (rng.standard_normal(100000) * 1e-39).astype(np.float32)    # binary32 subnormals
    v = np.concatenate([v, small, np.float32([3.4028235e38, -3.4028235e38])])
    got = oracle.float_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    b = np.arange(65536, dtype=np.uint16)
    back = oracle.bf16_to_float(b)
    tref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (back.view(np.uint32) == tref.view(np.uint32)) | (np.isnan(back) & np.isnan(tref))
    assert same.all()


# ---------------------------------------------------------------------------
# hand-derived fixtures
# ---------------------------------------------------------------------------

def test_worked_example_int4_group8():
    fx = _read_fixture("worked_int4_g8_f16.txt")
    bits, group = int(fx["bits"][0]), int(fx["group"][0])
    x = _f16([float(v) for v in fx["x"]]).reshape(1, 1, -1)
    codes1, s1, z1 = oracle.quantize_groups(x, oracle.F16, bits, group)
    assert int(s1[0, 0, 0]) == int(fx["s_bits"][0], 16)
    assert int(z1[0, 0, 0]) == int(fx["z_bits"][0], 16)
    assert list(_unpack(codes1, bits)[0, 0]) == [int(v) for v in fx["codes"]]
    assert list(codes1[0, 0]) == [int(v, 16) for v in fx["packed"]]
    out, o32 = oracle.dequantize(codes1[0], s1[0], z1[0], 1, 8, bits, group, oracle.F16,
                                 want_o32=True)
    assert list(o32[0].astype(np.float64)) == [float(v) for v in fx["dequant_f32"]]
    assert list(_hval(out[0])) == [float(v) for v in fx["out_f16"]]


def test_bf16_output_rounding_ties():
    fx = _read_fixture("dequant_bf16_ties.txt")
    bits, group = int(fx["bits"][0]), int(fx["group"][0])
    codes = np.array([[int(v) for v in fx["codes"]]], dtype=np.uint8)
    s = np.array([[int(fx["s_bits"][0], 16)]], dtype=np.uint16)
    z = np.array([[int(fx["z_bits"][0], 16)]], dtype=np.uint16)
    out, o32 = oracle.dequantize(codes, s, z, 1, group, bits, group, oracle.BF16, want_o32=True)
    assert list(o32[0].astype(np.float64)) == [float(v) for v in fx["o32"]]
    assert list(out[0]) == [int(v, 16) for v in fx["out_bf16_bits"]]


def test_sum_order_is_ascending_sequential():
    fx = _read_fixture("sum_order_r4.txt")
    vals = [float(v) for v in fx["values"]]
    R, T, H, g = 4, 1, 64, 16
    x = np.stack([np.full((T, H), _f16([v])[0], dtype=np.uint16) for v in vals])
    res = oracle.allreduce(x, oracle.F16, 8, g)
    assert np.all(res["s1"] == 0)                       # constant groups
    assert np.all(res["y"] == np.float32(float(fx["y_ascending"][0])))
    assert float(fx["y_pairwise"][0]) != float(fx["y_ascending"][0])
    # the fp64 sum differs too, so the fixture really discriminates
    assert sum(vals) != float(fx["y_ascending"][0])


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_constant_groups_round_trip_exactly(dtype):
    """Every group constant: s = 0, z = value, codes 0; sums of quarter-integers are exact."""
    rng = np.random.default_rng(3)
    R, T, H, g = 4, 6, 256, 32
    G = H // g
    vals = rng.integers(-32, 33, size=(R, T, G)).astype(np.float64) / 4.0
    x = np.repeat(vals, g, axis=2)
    xb = synth.operands_from_values(x, dtype)
    res = oracle.allreduce(xb, dtype, 8, g)
    assert np.all(res["s1"] == 0) and np.all(_unpack(res["codes1"], 8) == 0)
    wid = (lambda b: _hval(b)) if dtype == oracle.F16 else (
        lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64))
    assert np.array_equal(_hval(res["z1"]), vals)
    exact = x.sum(axis=0)
    assert np.array_equal(res["y"].astype(np.float64), exact)
    assert np.all(res["s2"] == 0) and np.all(_unpack(res["codes2"], 8) == 0)
    assert np.array_equal(wid(res["out"]), exact)


@pytest.mark.parametrize("bits", [4, 8])
def test_ramp_gives_codes_equal_to_index(bits):
    """x_i = a + i*d (d a power of two, i = 0..Q, any order): s = d, z = a, code of x_i is i."""
    rng = np.random.default_rng(bits)
    Q = 2 ** bits - 1
    g = Q + 1
    R, T, G = 2, 3, 2
    H = g * G
    x = np.empty((R, T, H))
    idx = np.empty((R, T, H), dtype=np.int64)
    ds = np.empty((R, T, G))
    As = np.empty((R, T, G))
    for r in range(R):
        for t in range(T):
            for k in range(G):
                d = 2.0 ** int(rng.integers(-8, -3))
                a = int(rng.integers(-64, 64)) * d
                perm = rng.permutation(g)
                x[r, t, k * g:(k + 1) * g] = a + perm * d
                idx[r, t, k * g:(k + 1) * g] = perm
                ds[r, t, k], As[r, t, k] = d, a
    codes, s, z = oracle.quantize_groups(_f16(x), oracle.F16, bits, g)
    assert np.array_equal(_unpack(codes, bits), idx)
    assert np.array_equal(_hval(s), ds)
    assert np.array_equal(_hval(z), As)


@pytest.mark.parametrize("bits,g", [(4, 6), (4, 24), (8, 96), (8, 258)])
def test_ramp_codes_in_groups_that_are_not_powers_of_two(bits, g):
    """Groups of any even length (here 6, 24, 96, 258 values): each group holds a + k*d for a
    set of levels k that includes 0 and Q (the rest drawn from [0, Q], any order), so s = d,
    z = a and every code is its k; the group boundaries and the scale/zero indices follow g."""
    rng = np.random.default_rng(g)
    Q = 2 ** bits - 1
    R, T, G = 2, 3, 4
    H = g * G
    x = np.empty((R, T, H))
    idx = np.empty((R, T, H), dtype=np.int64)
    ds = np.empty((R, T, G))
    As = np.empty((R, T, G))
    for r in range(R):
        for t in range(T):
            for k in range(G):
                d = 2.0 ** int(rng.integers(-8, -3))
                a = int(rng.integers(-64, 64)) * d
                lv = np.concatenate([[0, Q], rng.integers(0, Q + 1, size=g - 2)])
                lv = rng.permutation(lv)
                x[r, t, k * g:(k + 1) * g] = a + lv * d
                idx[r, t, k * g:(k + 1) * g] = lv
                ds[r, t, k], As[r, t, k] = d, a
    codes, s, z = oracle.quantize_groups(_f16(x), oracle.F16, bits, g)
    assert np.array_equal(_unpack(codes, bits), idx)
    assert np.array_equal(_hval(s), ds)
    assert np.array_equal(_hval(z), As)


def test_int4_nibble_order_even_element_low():
    x = _f16(np.arange(16) * 0.125).reshape(1, 1, 16)
    codes, s, z = oracle.quantize_groups(x, oracle.F16, 4, 16)
    assert list(codes[0, 0]) == [(2 * j) | ((2 * j + 1) << 4) for j in range(8)]


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_half_steps_round_to_even(bits):
    """Points exactly halfway between grid levels (power-of-two step) take the even code."""
    Q = 2 ** bits - 1
    g = Q + 1
    d = 2.0 ** -bits
    a = 1.0
    k = np.arange(Q - 1)
    vals = np.concatenate([[a, a + Q * d], a + (k + 0.5) * d])
    x = _f16(vals).reshape(1, 1, g)
    codes, s, z = oracle.quantize_groups(x, oracle.F16, bits, g)
    q = _unpack(codes, bits)[0, 0]
    assert q[0] == 0 and q[1] == Q
    expect = np.where(k % 2 == 0, k, k + 1)
    assert np.array_equal(q[2:], expect)


def test_bottom_clamp_when_zero_point_rounds_above_min():
    """fp32 sums near 1000 with range 0.01: fp16(min) = 1000.5 lies above every value -> codes 0."""
    v = np.float32([1000.3, 1000.31, 1000.305, 1000.3])
    for bits in (4, 8):
        codes, s, z = oracle.quantize_f32(v, bits, 4)
        assert _hval(z)[0] == 1000.5
        assert np.all(_unpack(codes[None], bits) == 0)


def test_top_clamp_with_subnormal_scale():
    """Values k * 2^-24, k = 0..14 and 21: s = fp16(1.4 * 2^-24) = 2^-24, so the code of k is min(k, 15)."""
    k = np.concatenate([np.arange(15), [21]])
    x = (k.astype(np.uint16)).reshape(1, 1, 16)          # fp16 subnormal bit patterns k
    codes, s, z = oracle.quantize_groups(x, oracle.F16, 4, 16)
    assert int(s[0, 0, 0]) == 1 and int(z[0, 0, 0]) == 0
    assert np.array_equal(_unpack(codes, 4)[0, 0], np.minimum(k, 15))


def test_zero_range_and_signed_zero_canonicalised():
    x = _f16([-0.0, 0.0, -0.0, 0.0, -0.0, -0.0, 0.0, 0.0]).reshape(1, 1, 8)
    x[0, 0, 0] = 0x8000
    codes, s, z = oracle.quantize_groups(x, oracle.F16, 8, 8)
    assert int(s[0, 0, 0]) == 0 and int(z[0, 0, 0]) == 0          # +0, never -0
    assert np.all(codes == 0)


def test_stage2_groups_are_min_of_group_and_chunk():
    """Stage-1 group spans the row (g = H); stage-2 groups are the R chunks of C = H/R columns."""
    R, T, H = 4, 2, 64
    C = H // R
    rng = np.random.default_rng(11)
    # operand 0 carries values on its stage-1 grid (codes 0..255 with both ends present);
    # operands 1..3 are 0, so y equals operand 0's dequantized values exactly.
    d, a = 2.0 ** -6, -2.0
    q = rng.integers(0, 256, size=(T, H))
    q[:, 0], q[:, 1] = 0, 255
    x = np.zeros((R, T, H))
    x[0] = a + q * d
    res = oracle.allreduce(_f16(x), oracle.F16, 8, H)
    assert res["group2"] == C and res["s2"].shape == (T, H // C)
    assert np.array_equal(res["y"].astype(np.float64), x[0])
    for t in range(T):
        for j in range(R):
            ch = x[0, t, j * C:(j + 1) * C]
            mn, mx = ch.min(), ch.max()
            s_exp = np.float32(np.float32(mx - mn) / np.float32(255)).astype(np.float16)
            assert _hval(res["s2"][t, j]) == float(s_exp)
            assert _hval(res["z2"][t, j]) == float(np.float16(mn))


def _fixture_group(name: str):
    fx = _read_fixture(name)
    bits, group = int(fx["bits"][0]), int(fx["group"][0])
    x = _f16([float(v) for v in fx["x"]]).reshape(1, 1, -1)
    codes1, s1, z1 = oracle.quantize_groups(x, oracle.F16, bits, group)
    return fx, bits, codes1, s1, z1


def test_codes_use_the_binary32_reciprocal_not_a_divide():
    """One element is an exact half step of (x - z)/s but not of fp32(x - z) * fp32(1/s):
    the pinned reading (one reciprocal per group) gives 15 where a divide gives 14."""
    fx, bits, codes1, s1, z1 = _fixture_group("recip_vs_divide_int4_g8_f16.txt")
    assert int(s1[0, 0, 0]) == int(fx["s_bits"][0], 16)
    assert int(z1[0, 0, 0]) == int(fx["z_bits"][0], 16)
    got = list(_unpack(codes1, bits)[0, 0])
    assert got == [int(v) for v in fx["codes"]]
    assert got != [int(v) for v in fx["codes_if_divided"]]
    assert list(codes1[0, 0]) == [int(v, 16) for v in fx["packed"]]


def test_codes_take_two_binary32_roundings():
    """t = fp32(fp32(x - z) * inv): six exact half steps round to the even codes, where one
    fused multiply-add on the distributed form x*inv - z*inv rounds them to the odd ones."""
    fx, bits, codes1, s1, z1 = _fixture_group("two_roundings_int4_g8_f16.txt")
    assert int(s1[0, 0, 0]) == int(fx["s_bits"][0], 16)
    assert int(z1[0, 0, 0]) == int(fx["z_bits"][0], 16)
    got = list(_unpack(codes1, bits)[0, 0])
    assert got == [int(v) for v in fx["codes"]]
    assert got != [int(v) for v in fx["codes_if_fused"]]
    assert list(codes1[0, 0]) == [int(v, 16) for v in fx["packed"]]


def test_scale_is_the_binary32_quotient_of_the_range():
    """range/Q is exactly an fp16 tie (ties to even: 0x360E); the range times the
    binary32 reciprocal of Q lies above the tie and would store 0x360F."""
    fx, bits, codes1, s1, z1 = _fixture_group("scale_is_a_quotient_int4_g8_f16.txt")
    assert int(s1[0, 0, 0]) == int(fx["s_bits"][0], 16)
    assert int(s1[0, 0, 0]) != int(fx["s_bits_if_reciprocal"][0], 16)
    assert int(z1[0, 0, 0]) == int(fx["z_bits"][0], 16)
    assert list(_unpack(codes1, bits)[0, 0]) == [int(v) for v in fx["codes"]]
    assert list(codes1[0, 0]) == [int(v, 16) for v in fx["packed"]]


def test_stage2_zero_point_below_the_minimum():
    """A stage-2 group whose minimum sum is a tie in fp16 that rounds below it: z2 lies
    under the group, the top code clamps at Q, and that element's error is a whole scale
    step -- over s/2, within s/2 + |z - min|. The other chunk is reproduced exactly."""
    fx = _read_fixture("stage2_zero_below_min_r2_int4.txt")
    bits, group = int(fx["bits"][0]), int(fx["group"][0])
    x = np.stack([_f16([float(v) for v in fx["x0"]]), _f16([float(v) for v in fx["x1"]])])
    x = x.reshape(2, 1, -1)
    res = oracle.allreduce(x, oracle.F16, bits, group)
    hexes = lambda k: [int(v, 16) for v in fx[k]]
    assert list(res["s1"][0, 0]) == hexes("s1_bits_r0")
    assert list(res["z1"][0, 0]) == hexes("z1_bits_r0")
    assert list(res["s1"][1, 0]) == hexes("s1_bits_r1")
    assert list(res["z1"][1, 0]) == hexes("z1_bits_r1")
    assert list(_unpack(res["codes1"], bits)[1, 0]) == [int(v) for v in fx["codes1_r1"]]
    assert not _unpack(res["codes1"], bits)[0].any()
    y = res["y"][0].astype(np.float64)
    assert list(y) == [float(v) for v in fx["y"]]
    assert res["group2"] == 8
    assert list(res["s2"][0]) == hexes("s2_bits")
    assert list(res["z2"][0]) == hexes("z2_bits")
    assert list(_unpack(res["codes2"], bits)[0]) == [int(v) for v in fx["codes2"]]
    assert list(res["codes2"][0]) == hexes("packed2")
    o32 = res["o32"][0].astype(np.float64)
    assert list(o32) == [float(v) for v in fx["o32"]]
    assert list(_hval(res["out"][0])) == [float(v) for v in fx["out_f16"]]
    s2 = _hval(res["s2"][0])
    z2 = _hval(res["z2"][0])
    err = np.abs(o32 - y).reshape(2, 8).max(axis=1)
    mn = y.reshape(2, 8).min(axis=1)
    assert err[0] == s2[0] > s2[0] / 2          # the clamp: more than half a scale
    assert err[0] <= s2[0] / 2 + abs(z2[0] - mn[0])
    assert err[1] == 0.0


# ---------------------------------------------------------------------------
# brute force: the code is the nearest grid point
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_codes_are_nearest_grid_point_exhaustive(bits):
    """For ~50 (mn, mx) pairs, every fp16 value between them: |q - (x - z)/s| <= 1/2 + eps,
    q is the nearest level whenever the distance to a tie exceeds eps, and s, z are the
    fp16 roundings of (mx - mn)/Q and mn."""
    rng = np.random.default_rng(100 + bits)
    Q = 2 ** bits - 1
    eps = (Q + 1) * 4.0 * 2.0 ** -24
    g = 64
    for _ in range(50):
        e = int(rng.integers(-6, 4))
        mn = float(np.float16(rng.uniform(-1, 1) * 2.0 ** e))
        mx = float(np.float16(mn + abs(rng.uniform(0.01, 1)) * 2.0 ** e))
        if mx <= mn:
            continue
        lo = np.float16(mn).view(np.uint16)
        # all fp16 values in [mn, mx]
        allh = np.arange(65536, dtype=np.uint16)
        allv = allh.view(np.float16).astype(np.float64)
        inside = allv[np.isfinite(allv) & (allv >= mn) & (allv <= mx)]
        inside = np.unique(inside)
        n_per = g - 2
        pad = (-inside.size) % n_per
        body = np.concatenate([inside, np.full(pad, mn)]).reshape(-1, n_per)
        grp = np.concatenate([np.full((body.shape[0], 1), mn), np.full((body.shape[0], 1), mx),
                              body], axis=1)
        x = _f16(grp).reshape(1, body.shape[0], g)
        codes, s, z = oracle.quantize_groups(x, oracle.F16, bits, g)
        q = _unpack(codes, bits)[0].astype(np.float64)
        sv = _hval(s)[0]
        zv = _hval(z)[0]
        assert np.all(zv == mn), lo
        s_true = (mx - mn) / Q
        half_spacing = 0.5 * max(2.0 ** (np.floor(np.log2(s_true)) - 10), 2.0 ** -24)
        assert np.all(np.abs(sv - s_true) <= half_spacing + s_true * 2.0 ** -23)
        u = np.clip((grp - zv) / sv, 0, Q)        # out-of-grid points clamp to the end level
        assert np.all((q >= 0) & (q <= Q))
        assert np.all(np.abs(q - u) <= 0.5 + eps)
        far = np.abs(np.abs(u - np.floor(u)) - 0.5) > eps
        nearest = np.clip(np.floor(u + 0.5), 0, Q)
        assert np.array_equal(q[far], nearest[far])


# ---------------------------------------------------------------------------
# bounds, symmetries and statistics
# ---------------------------------------------------------------------------

def _small(name: str, T: int = 64, **kw) -> synth.Workload:
    return synth.workload(name).with_(T=T, **kw)


_BOUND_CASES = ["tiny", "llama3_8b_prefill", "llama3_70b_prefill", "decode",
                "sweep_int8_g4096", "sweep_int4_g4096", "sweep_int8_g1024", "sweep_int4_g256"]


def _widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == oracle.F16:
        return _hval(bits)
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name", _BOUND_CASES)
def test_per_stage_error_at_most_half_scale(name):
    """|x_hat - x| <= s*(1/2 + 2^-14) + 2^-23*|x| + |z - mn| per stage (normal scales).
    The last term is the distance of the fp16 zero point from the group minimum: 0 for
    fp16 stage-1 input, up to half an fp16 spacing of |mn| for binary32 stage-2 sums,
    where a zero below the minimum clamps the top codes at Q."""
    w = _small(name, T=16)
    x = synth.operands(w, 0)
    res = oracle.allreduce(x, w.dtype, w.bits, w.group)
    R, T, H = x.shape
    g, g2 = w.group, res["group2"]
    # stage 1
    xv = _widen(x, w.dtype).reshape(R, T, H // g, g)
    q1 = _unpack(res["codes1"], w.bits).reshape(R, T, H // g, g).astype(np.float64)
    s1 = _hval(res["s1"])[..., None]
    z1 = _hval(res["z1"])[..., None]
    xh = (q1 * s1 + z1).astype(np.float32).astype(np.float64)
    mn = xv.min(axis=-1, keepdims=True)
    bound = s1 * (0.5 + 2.0 ** -14) + 2.0 ** -23 * np.abs(xv) + np.abs(z1 - mn)
    normal = s1 >= 2.0 ** -14
    assert np.all((np.abs(xh - xv) <= bound) | ~normal)
    # stage 2 against its own input y
    y = res["y"].astype(np.float64).reshape(T, H // g2, g2)
    o = res["o32"].astype(np.float64).reshape(T, H // g2, g2)
    s2 = _hval(res["s2"])[..., None]
    z2 = _hval(res["z2"])[..., None]
    mn2 = y.min(axis=-1, keepdims=True)
    bound2 = s2 * (0.5 + 2.0 ** -14) + 2.0 ** -23 * np.abs(y) + np.abs(z2 - mn2)
    assert np.all((np.abs(o - y) <= bound2) | ~(s2 >= 2.0 ** -14))


def test_stage2_bound_needs_the_zero_point_term():
    """Groups with a large offset and a small range (R = 2, fp16, 4-bit codes, groups of 32):
    the stage-2 error stays within s/2 + |z - mn| everywhere, and the |z - mn| term is
    needed -- without it the bound fails where the fp16 zero rounds below the minimum sum."""
    rng = np.random.default_rng(11)
    R, T, H, g = 2, 16, 256, 32
    off = rng.uniform(-60, -35, size=(1, T, H // g, 1))
    v = off / R + rng.uniform(-0.02, 0.02, size=(R, T, H // g, g))
    x = v.reshape(R, T, H).astype(np.float16).view(np.uint16)
    res = oracle.allreduce(x, oracle.F16, 4, g)
    y = res["y"].astype(np.float64).reshape(T, H // g, g)
    o = res["o32"].astype(np.float64).reshape(T, H // g, g)
    s2 = _hval(res["s2"])[..., None]
    z2 = _hval(res["z2"])[..., None]
    mn2 = y.min(axis=-1, keepdims=True)
    err = np.abs(o - y)
    half = s2 * (0.5 + 2.0 ** -14) + 2.0 ** -23 * np.abs(y)
    assert np.all(err <= half + np.abs(z2 - mn2))
    assert np.any(err > half)


@pytest.mark.parametrize("name", _BOUND_CASES)
def test_end_to_end_error_within_stated_tolerance(name):
    """|o32 - sum_r x_r| <= sum_r s1_r/2 + s2/2 + 2^-10 |sum_r x_r| (exact sum in fp64)."""
    w = _small(name, T=16)
    x = synth.operands(w, 1)
    res = oracle.allreduce(x, w.dtype, w.bits, w.group)
    R, T, H = x.shape
    exact = _widen(x, w.dtype).sum(axis=0)
    s1 = np.repeat(_hval(res["s1"]), w.group, axis=2).sum(axis=0)
    s2 = np.repeat(_hval(res["s2"]), res["group2"], axis=1)
    tol = s1 / 2 + s2 / 2 + 2.0 ** -10 * np.abs(exact)
    assert np.all(np.abs(res["o32"].astype(np.float64) - exact) <= tol)
    out = _widen(res["out"], w.dtype)
    ulp_half = np.abs(exact) * (2.0 ** -11 if w.dtype == oracle.F16 else 2.0 ** -8)
    assert np.all(np.abs(out - exact) <= tol + ulp_half + 2.0 ** -24)


def test_two_operands_commute():
    w = _small("llama3_8b_prefill", T=8, R=2)
    x = synth.operands(w, 5)
    a = oracle.allreduce(x, w.dtype, w.bits, w.group)
    b = oracle.allreduce(x[::-1].copy(), w.dtype, w.bits, w.group)
    for k in ("codes2", "s2", "z2", "out"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("factor", [2.0, 0.5])
def test_scaling_by_power_of_two_is_equivariant(factor):
    w = _small("llama3_8b_prefill", T=8)
    x = synth.operands(w, 2)
    xv = _hval(x)
    xv = xv[np.newaxis] if xv.ndim == 2 else xv
    keep = np.abs(xv) >= 2.0 ** -12                   # stay clear of fp16 subnormals
    xv = np.where(keep, xv, 0.25)
    a = oracle.allreduce(_f16(xv), w.dtype, w.bits, w.group)
    b = oracle.allreduce(_f16(xv * factor), w.dtype, w.bits, w.group)
    for k in ("codes1", "codes2"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("s1", "z1", "s2", "z2"):
        assert np.array_equal(_hval(a[k]) * factor, _hval(b[k])), k


def test_single_operand_stage2_requantizes_stage1_values():
    w = _small("llama3_8b_prefill", T=4, R=1, H=1024)
    x = synth.operands(w, 3)
    res = oracle.allreduce(x, w.dtype, w.bits, w.group)
    xh, _ = oracle.dequantize(res["codes1"][0], res["s1"][0], res["z1"][0], w.T, w.H, w.bits,
                              w.group, oracle.F16, want_o32=True)
    _, o32 = oracle.dequantize(res["codes1"][0], res["s1"][0], res["z1"][0], w.T, w.H, w.bits,
                               w.group, oracle.F16, want_o32=True)
    assert np.array_equal(res["y"], o32)
    c, s, z = oracle.quantize_f32(o32, w.bits, w.group)
    assert np.array_equal(c.reshape(w.T, -1), res["codes2"])
    assert np.array_equal(s.reshape(w.T, -1), res["s2"])


@pytest.mark.parametrize("bits", [4, 8])
def test_stage1_mse_matches_uniform_error_model(bits):
    """Rounding error uniform over a step: MSE ~ mean(s^2)/12 (no outliers, Gaussian data)."""
    w = _small("llama3_8b_prefill", T=64, bits=bits, outlier_frac=0.0)
    x = synth.operands(w, 9)
    res = oracle.allreduce(x, w.dtype, w.bits, w.group)
    R, T, H = x.shape
    xv = _hval(x)
    q1 = _unpack(res["codes1"], bits).astype(np.float64)
    s1 = np.repeat(_hval(res["s1"]), w.group, axis=2)
    z1 = np.repeat(_hval(res["z1"]), w.group, axis=2)
    mse = np.mean((q1 * s1 + z1 - xv) ** 2)
    model = np.mean(_hval(res["s1"]) ** 2) / 12.0
    assert abs(mse / model - 1.0) < 0.10


def test_mse_falls_with_finer_groups_and_more_bits():
    """Figure 4: finer blocks (4096 -> 128) quantize activations more accurately; and 8-bit
    codes beat 4-bit codes at every block size. Checked on stage-1 and end-to-end MSE."""
    mse = {}
    for bits in synth.SWEEP_BITS:
        for g in synth.SWEEP_GROUPS:
            w = _small(f"sweep_int{bits}_g{g}", T=32)
            x = synth.operands(w, 0)
            res = oracle.allreduce(x, w.dtype, w.bits, w.group)
            exact = _hval(x).sum(axis=0)
            mse[bits, g] = float(np.mean((res["o32"].astype(np.float64) - exact) ** 2))
    for bits in synth.SWEEP_BITS:
        seq = [mse[bits, g] for g in synth.SWEEP_GROUPS]
        assert all(a > b for a, b in zip(seq, seq[1:])), (bits, seq)
    for g in synth.SWEEP_GROUPS:
        assert mse[4, g] > mse[8, g]


# ---------------------------------------------------------------------------
# argument checks and out-of-contract input
# ---------------------------------------------------------------------------

def test_rejects_invalid_arguments():
    x = np.zeros((2, 1, 64), dtype=np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_groups(x, oracle.F16, 5, 16)          # bits
    with pytest.raises(oracle.OracleError):
        oracle.quantize_groups(x, oracle.F16, 4, 24)          # group does not divide H
    with pytest.raises(oracle.OracleError):
        oracle.dequant_sum_requant(np.zeros((3, 1, 32), np.uint8), np.zeros((3, 1, 4), np.uint16),
                                   np.zeros((3, 1, 4), np.uint16), 3, 1, 64, 4, 16)   # H % R


def test_rejects_fp16_overflowing_zero_point():
    x = np.full((1, 1, 8), 0x7BFF, dtype=np.uint16)           # fp16 max is fine
    oracle.quantize_groups(x, oracle.F16, 8, 8)
    xb = synth.operands_from_values(np.full((1, 1, 8), 70000.0), oracle.BF16)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_groups(xb, oracle.BF16, 8, 8)


def test_empty_token_dimension():
    x = np.zeros((2, 0, 64), dtype=np.uint16)
    res = oracle.allreduce(x, oracle.F16, 4, 16)
    assert res["out"].shape == (0, 64)


# ---------------------------------------------------------------------------
# the uncompressed comparator (the ring all-reduce's result)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_uncompressed_sum_exact_for_dyadic_operands(dtype):
    """Quarter-integers in [-8, 8]: every partial sum is exact in binary32 and the total fits
    the 16-bit type, so the result is the exact sum (closed form)."""
    rng = np.random.default_rng(21)
    x = rng.integers(-32, 33, size=(4, 5, 64)) / 4.0
    out = oracle.sum_uncompressed(synth.operands_from_values(x, dtype), dtype)
    assert np.array_equal(_widen(out, dtype), x.sum(axis=0))


def test_uncompressed_sum_is_rounded_exact_sum_for_two_operands():
    """R = 2: the binary32 sum of two fp16 values is within 2^-24 (relative) of the exact sum,
    so rounding it to fp16 gives numpy's float16 rounding of the fp64 sum unless the binary32
    rounding lands exactly on an fp16 midpoint (this data has no such case); swapping the
    operands changes nothing."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((2, 16, 256)) * 4).astype(np.float16)
    xb = x.view(np.uint16)
    out = oracle.sum_uncompressed(xb, oracle.F16)
    exact = x.astype(np.float64).sum(axis=0)
    assert np.array_equal(out, exact.astype(np.float16).view(np.uint16))
    assert np.array_equal(out, oracle.sum_uncompressed(xb[::-1].copy(), oracle.F16))


def test_uncompressed_sum_accumulates_in_binary32_ascending():
    """Three operands: 1 + 2^-24 ties to 1 in binary32, so the ascending sum is +0, where the
    exact sum and the descending order both give the subnormal 2^-24."""
    fx = _read_fixture("uncompressed_sum_r3_f16.txt")
    x = np.stack([_f16([float(v) for v in fx[k]]) for k in ("x0", "x1", "x2")]).reshape(3, 1, 2)
    assert int(x[1, 0, 0]) == 0x0001
    out = oracle.sum_uncompressed(x, oracle.F16)
    hexes = lambda k: [int(v, 16) for v in fx[k]]
    assert list(out[0]) == hexes("out_bits")
    assert list(out[0]) != hexes("out_bits_if_exact")
    assert list(out[0]) != hexes("out_bits_if_descending")


def test_uncompressed_sum_error_bound():
    """|out - sum| <= (R-1) * 2^-24 * sum|x| + half a 16-bit ulp (sequential binary32 sum, one rounding)."""
    w = _small("llama3_70b_prefill", T=8)
    x = synth.operands(w, 4)
    out = _widen(oracle.sum_uncompressed(x, w.dtype), w.dtype)
    xv = _widen(x, w.dtype)
    exact = xv.sum(axis=0)
    bound = (w.R - 1) * 2.0 ** -24 * np.abs(xv).sum(axis=0) + np.abs(exact) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(out - exact) <= bound)


# ---------------------------------------------------------------------------
# different code widths before the reduce-scatter and before the all-gather
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,bits2", [(4, 8), (8, 4)])
def test_mixed_widths_constant_groups_round_trip(bits, bits2):
    rng = np.random.default_rng(31)
    R, T, H, g = 4, 3, 256, 32
    vals = rng.integers(-32, 33, size=(R, T, H // g)) / 4.0
    x = np.repeat(vals, g, axis=2)
    res = oracle.allreduce(_f16(x), oracle.F16, bits, g, bits2=bits2)
    assert res["codes2"].shape == (T, H * bits2 // 8)
    assert np.array_equal(_hval(res["out"]), x.sum(axis=0))


@pytest.mark.parametrize("bits,bits2", [(4, 8), (8, 4)])
def test_mixed_widths_error_bound(bits, bits2):
    """|o32 - sum x| <= sum_r s1_r/2 + s2/2 + 2^-10 |sum x| with each stage's own scale."""
    w = _small("llama3_8b_prefill", T=16)
    x = synth.operands(w, 8)
    res = oracle.allreduce(x, w.dtype, bits, w.group, bits2=bits2)
    exact = _widen(x, w.dtype).sum(axis=0)
    s1 = np.repeat(_hval(res["s1"]), w.group, axis=2).sum(axis=0)
    s2 = np.repeat(_hval(res["s2"]), res["group2"], axis=1)
    tol = s1 / 2 + s2 / 2 + 2.0 ** -10 * np.abs(exact)
    assert np.all(np.abs(res["o32"].astype(np.float64) - exact) <= tol)


def test_mixed_widths_mse_between_uniform_widths():
    """Figure 5 (right) contrasts the error of quantizing before RS and before AG: 8 bits at
    either step lowers the end-to-end MSE of all-4-bit codes, and all-8-bit codes are best."""
    w = _small("llama3_8b_prefill", T=32)
    x = synth.operands(w, 12)
    exact = _hval(x).sum(axis=0)
    mse = {}
    for b1 in (4, 8):
        for b2 in (4, 8):
            o = oracle.allreduce(x, w.dtype, b1, w.group, bits2=b2)["o32"].astype(np.float64)
            mse[b1, b2] = float(np.mean((o - exact) ** 2))
    assert mse[4, 4] > mse[4, 8] > mse[8, 8]
    assert mse[4, 4] > mse[8, 4] > mse[8, 8]


# ---------------------------------------------------------------------------
# the final dequantize fused with the residual add (Figure 3's block)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fixture", ["residual_add_f16.txt", "residual_add_bf16.txt"])
def test_residual_add_rounds_the_allreduce_result_first(fixture):
    fx = _read_fixture(fixture)
    bits, group, dt = int(fx["bits"][0]), int(fx["group"][0]), fx["dtype"][0]
    codes = np.array([[int(v) for v in fx["codes"]]], dtype=np.uint8)
    s = np.array([[int(fx["s_bits"][0], 16)]], dtype=np.uint16)
    z = np.array([[int(fx["z_bits"][0], 16)]], dtype=np.uint16)
    res = np.array([[int(v, 16) for v in fx["residual_bits"]]], dtype=np.uint16)
    a, _ = oracle.dequantize(codes, s, z, 1, group, bits, group, dt)
    assert list(a[0]) == [int(v, 16) for v in fx["a_bits"]]
    out = oracle.dequantize_residual(codes, s, z, 1, group, bits, group, dt, res)
    assert list(out[0]) == [int(v, 16) for v in fx["out_bits"]]


def _payload_and_residual(dtype: str, bits: int, seed: int):
    w = synth.workload("tiny").with_(dtype=dtype, bits=bits, T=16, H=512, R=4, group=128)
    x = synth.operands(w, seed)
    ref = oracle.allreduce(x, dtype, bits, w.group, want_f32=False)
    # the residual stream: another seeded activation of the same shape
    residual = synth.operands(w.with_(R=1, sigma=4.0), seed + 1000)[0]
    return w, ref, residual


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("bits", [4, 8])
def test_residual_add_equals_torch_add_of_the_two_steps(dtype, bits):
    """Library routine: torch's CPU add of two 16-bit tensors (binary32 add, one
    rounding) applied to the residual and the separately dequantized result."""
    w, ref, residual = _payload_and_residual(dtype, bits, seed=5)
    out = oracle.dequantize_residual(ref["codes2"], ref["s2"], ref["z2"], w.T, w.H, bits,
                                     ref["group2"], dtype, residual)
    tdt = torch.float16 if dtype == oracle.F16 else torch.bfloat16
    a = torch.from_numpy(ref["out"].view(np.int16)).view(tdt)
    r = torch.from_numpy(residual.view(np.int16)).view(tdt)
    expect = (r + a).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_residual_add_closed_forms(dtype):
    w, ref, _ = _payload_and_residual(dtype, 4, seed=6)
    args = (ref["codes2"], ref["s2"], ref["z2"], w.T, w.H, 4, ref["group2"], dtype)
    a = ref["out"]
    # +0 residual: the all-reduce result itself (as a value; -0 + +0 is +0)
    out0 = oracle.dequantize_residual(*args, np.zeros_like(a))
    widen = oracle.half_to_float if dtype == oracle.F16 else oracle.bf16_to_float
    assert np.array_equal(widen(out0), widen(a))
    # residual = -result: every element cancels to +0
    neg = oracle.dequantize_residual(*args, a ^ np.uint16(0x8000))
    assert np.all(neg == 0)


# ---------------------------------------------------------------------------
# the row-parallel linear layer that produces the all-reduce operands (Figure 3)
# ---------------------------------------------------------------------------

def _dyadic(rng, shape, lo, hi, exp):
    """Integers k in [lo, hi] scaled by 2^exp, as float64, and the integers."""
    k = rng.integers(lo, hi + 1, size=shape).astype(np.int64)
    return k, k.astype(np.float64) * 2.0 ** exp


def _to_dtype_bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """Library rounding of float64 values exact in binary32: numpy's float16, torch's bfloat16."""
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)
    if dtype == oracle.F16:
        return v32.astype(np.float16).view(np.uint16)
    return torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_linear_matches_integer_matmul(dtype):
    """Integer arithmetic: with dyadic inputs every product and partial sum is an
    integer multiple of 2^-9 below 2^24 of those units, so the layer output is
    the int64 matmul, scaled, and rounded once to the dtype. Non-square shapes
    and R > 1 catch a transposed or mismatched operand."""
    rng = np.random.default_rng(21)
    R, T, K, H = 3, 5, 24, 40
    ka, af = _dyadic(rng, (R, T, K), -8, 8, -3)
    kw, wf = _dyadic(rng, (R, H, K), -8, 8, -6)
    kw[:, 7] *= 16                                 # an outlier output channel
    wf[:, 7] *= 16
    a = _to_dtype_bits(af, dtype)
    w = _to_dtype_bits(wf, dtype)
    exact = np.einsum("rtk,rhk->rth", ka, kw).astype(np.float64) * 2.0 ** -9
    y = oracle.linear(a, w, dtype)
    assert y.shape == (R, T, H)
    assert np.array_equal(y, _to_dtype_bits(exact, dtype))


def test_linear_permutation_weight_gathers_columns():
    """Closed form: a weight with one 1 per output row (w[n][pi(n)] = 1) copies
    input column pi(n) to output column n."""
    rng = np.random.default_rng(22)
    T, K = 6, 16
    pi = rng.permutation(K)
    a = synth.operands_from_values(rng.normal(size=(1, T, K)), oracle.BF16)
    w = np.zeros((1, K, K), dtype=np.uint16)
    w[0, np.arange(K), pi] = 0x3F80                # bfloat16 1.0
    y = oracle.linear(a, w, oracle.BF16)
    assert np.array_equal(y[0], a[0][:, pi])


def test_linear_quantize_codes_are_those_of_the_layer_output():
    rng = np.random.default_rng(23)
    R, T, K, H = 2, 4, 32, 256
    a = synth.operands_from_values(rng.normal(size=(R, T, K)), oracle.BF16)
    w = synth.operands_from_values(rng.normal(size=(R, H, K)) * 0.05, oracle.BF16)
    got = oracle.linear_quantize(a, w, oracle.BF16, 4, 128)
    # the codes dequantize to within half a scale of the layer output (stage-1 bound)
    y = oracle.bf16_to_float(got["y"]).astype(np.float64)
    s = _hval(got["s1"]).repeat(128, axis=-1)
    z = _hval(got["z1"]).repeat(128, axis=-1)
    q = _unpack(got["codes1"], 4).astype(np.float64)
    assert np.all(np.abs(q * s + z - y) <= s * (0.5 + 2.0 ** -14) + 2.0 ** -23 * np.abs(y)
                  + np.maximum(0.0, z - y.reshape(R, T, -1, 128).min(-1).repeat(128, -1)))

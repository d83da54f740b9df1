"""Seeded synthetic activations for the low-bit all-reduce codec.

This module only draws inputs: it holds none of the codec's arithmetic, so the
CPU oracle and the GPU path can both take their operands from it.

Every value comes from a counter-based generator (SplitMix64, Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) keyed by
(seed, stream) and indexed by the element's flat position, so any slice of an
operand tensor can be drawn on its own and is identical to the same slice of a
full draw.

Workloads stand in for the tensor-parallel all-reduce operands of the Flash
Communication page (Figure 1: LLaMA-3-70B prefill, batch 8 x 1024 tokens,
TP=4; Figure 4: LLaMA-3-8B with quantization blocks from 4096 down to 128).
The pages print no activation statistics, so values are Gaussian or Laplace
with a few hidden channels scaled up as outliers.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "operands", "operands_from_values",
    "outlier_channels", "uniform", "checksum", "F16", "BF16",
]

F16 = "f16"
BF16 = "bf16"

_GOLDEN = 0x9E3779B97F4A7C15
_STREAM_MUL = 0xD1B54A32D192ED03
_M64 = (1 << 64) - 1

STREAM_VALUES = 0
STREAM_OUTLIERS = 1

_CHUNK = 1 << 21


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, arithmetic parameters and value recipe of one set of operands."""

    name: str
    R: int                  # number of partial-sum operands (TP ranks)
    T: int                  # tokens
    H: int                  # hidden size
    dtype: str              # "f16" or "bf16"
    bits: int               # code width, 4 or 8
    group: int              # stage-1 group length along the hidden dimension
    dist: str = "normal"    # "normal" or "laplace"
    sigma: float = 1.0      # standard deviation of the normal draw
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    ffn: int = 0            # MLP intermediate size of the model (0: not a model shape)

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.H))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BASE = {
    "tiny": Workload("tiny", R=2, T=8, H=256, dtype=F16, bits=8, group=128),
    "llama3_8b_prefill": Workload(
        "llama3_8b_prefill", R=4, T=8192, H=4096, dtype=F16, bits=4, group=128,
        outlier_frac=0.01, outlier_scale=20.0, ffn=14336),
    "llama3_70b_prefill": Workload(
        "llama3_70b_prefill", R=4, T=8192, H=8192, dtype=BF16, bits=4, group=128,
        sigma=0.5, outlier_frac=0.005, outlier_scale=30.0, ffn=28672),
    "decode": Workload(
        "decode", R=8, T=64, H=8192, dtype=BF16, bits=4, group=128, dist="laplace",
        ffn=28672),
}
SWEEP_GROUPS = (4096, 1024, 512, 256, 128)
SWEEP_BITS = (8, 4)
for _b in SWEEP_BITS:
    for _g in SWEEP_GROUPS:
        _BASE[f"sweep_int{_b}_g{_g}"] = Workload(
            f"sweep_int{_b}_g{_g}", R=4, T=4096, H=4096, dtype=F16, bits=_b, group=_g,
            outlier_frac=0.01, outlier_scale=20.0)

WORKLOADS = dict(_BASE)


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on uint64 arrays (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> int:
    z = (int(seed) * _GOLDEN + int(stream) * _STREAM_MUL + 1) & _M64
    return int(_mix(np.array([z], dtype=np.uint64))[0])


def _raw(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """The idx-th SplitMix64 output of the generator keyed by (seed, stream)."""
    key = np.uint64(_key(seed, stream))
    with np.errstate(over="ignore"):
        state = key + (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(_GOLDEN)
        return _mix(state)


def uniform(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Uniform doubles in the open interval (0, 1) from the top 53 bits."""
    r = _raw(seed, stream, idx) >> np.uint64(11)
    return (r.astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal(seed: int, idx: np.ndarray) -> np.ndarray:
    """Box-Muller: element i takes the cosine (even i) or sine (odd i) branch of pair i // 2."""
    pair = idx >> 1
    u1 = uniform(seed, STREAM_VALUES, 2 * pair)
    u2 = uniform(seed, STREAM_VALUES, 2 * pair + 1)
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * math.pi * u2
    return np.where((idx & 1) == 0, rad * np.cos(ang), rad * np.sin(ang))


def _laplace(seed: int, idx: np.ndarray) -> np.ndarray:
    """Laplace(0, 1) by the inverse CDF."""
    u = uniform(seed, STREAM_VALUES, idx) - 0.5
    return -np.sign(u) * np.log1p(-2.0 * np.abs(u))


def outlier_channels(seed: int, H: int, count: int) -> np.ndarray:
    """`count` distinct hidden channels chosen by a partial Fisher-Yates shuffle."""
    perm = np.arange(H, dtype=np.int64)
    if count <= 0:
        return perm[:0]
    u = uniform(seed, STREAM_OUTLIERS, np.arange(count, dtype=np.int64))
    for i in range(count):
        j = i + int(u[i] * (H - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def _round_to_dtype(v32: np.ndarray, dtype: str) -> np.ndarray:
    """Round binary32 values to the 16-bit format (nearest, ties to even); returns the bit patterns."""
    if dtype == F16:
        return v32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        b = v32.view(np.uint32)
        b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
        return (b >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _fill(w: Workload, seed: int, out: np.ndarray, flat_start: int, scale_ch: np.ndarray) -> None:
    n = out.size
    idx = np.arange(flat_start, flat_start + n, dtype=np.int64)
    if w.dist == "normal":
        v = _normal(seed, idx)
    elif w.dist == "laplace":
        v = _laplace(seed, idx)
    else:
        raise ValueError(w.dist)
    v32 = v.astype(np.float32) * np.float32(w.sigma)
    h = idx % w.H
    v32 = v32 * scale_ch[h]
    out[...] = _round_to_dtype(v32, w.dtype)


def operands(w: Workload, seed: int, tokens: slice | None = None, threads: int | None = None) -> np.ndarray:
    """Bit patterns (uint16) of the R operands, shape [R, T', H] for the token slice `tokens`.

    Element (r, t, h) is drawn at flat position (r*T + t)*H + h, whatever the slice.
    """
    t0, t1, step = (tokens or slice(0, w.T)).indices(w.T)
    if step != 1:
        raise ValueError("token slice must be contiguous")
    nt = t1 - t0
    out = np.empty((w.R, nt, w.H), dtype=np.uint16)
    scale_ch = np.ones(w.H, dtype=np.float32)
    scale_ch[outlier_channels(seed, w.H, w.n_outliers)] = np.float32(w.outlier_scale)
    jobs = []
    for r in range(w.R):
        flat = out[r].reshape(-1)
        base = (r * w.T + t0) * w.H
        for s in range(0, flat.size, _CHUNK):
            jobs.append((flat[s:s + _CHUNK], base + s))
    if threads is None:
        threads = min(8, os.cpu_count() or 1)
    if threads <= 1 or len(jobs) <= 1:
        for dst, start in jobs:
            _fill(w, seed, dst, start, scale_ch)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda j: _fill(w, seed, j[0], j[1], scale_ch), jobs))
    return out


def operands_from_values(values: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of hand-built operand values (any float array), rounded to the 16-bit dtype."""
    return _round_to_dtype(np.asarray(values, dtype=np.float32), dtype)


def checksum(a: np.ndarray) -> str:
    """64-bit BLAKE2b digest of an array's bytes, for logs."""
    return hashlib.blake2b(np.ascontiguousarray(a).tobytes(), digest_size=8).hexdigest()

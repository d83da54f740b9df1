"""Second, vectorised numpy statement of the codec, used only to cross-check the
C oracle on medium sizes (it is a re-derivation, not a pin on its own).

Arithmetic: numpy float32 operations (each rounded to nearest even, never
fused), np.rint (ties to even), numpy's float16 conversion for fp16 rounding,
and a bit-level round-half-to-even for bfloat16. Unlike the oracle, it works
on the flat [rows, groups, group] view: the hidden chunks of the
reduce-scatter only show up through the stage-2 group length min(group, H/R).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    b = np.asarray(v, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def narrow(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(v)


def quantize(v: np.ndarray, bits: int):
    """v: float32 [..., G, g] -> (codes u8 [..., G, g], s16 bits, z16 bits [..., G])."""
    Q = np.float32(2 ** bits - 1)
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    mn = np.where(mn == 0, np.float32(0), mn).astype(np.float32)
    mx = np.where(mx == 0, np.float32(0), mx).astype(np.float32)
    s32 = (mx - mn) / Q
    s16 = s32.astype(np.float16)
    z16 = mn.astype(np.float16)
    s = s16.astype(np.float32)
    z = z16.astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(s == 0, np.float32(0), np.float32(1) / s).astype(np.float32)
    t = (v - z[..., None]) * inv[..., None]
    q = np.clip(np.rint(t), 0, Q).astype(np.uint8)
    return q, s16.view(np.uint16), z16.view(np.uint16)


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    q = q.reshape(q.shape[0], -1) if q.ndim > 1 else q[None]
    if bits == 8:
        return q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack(c: np.ndarray, bits: int) -> np.ndarray:
    if bits == 8:
        return c
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


def dequant(q: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray) -> np.ndarray:
    s = s_bits.view(np.float16).astype(np.float32)
    z = z_bits.view(np.float16).astype(np.float32)
    return q.astype(np.float32) * s[..., None] + z[..., None]


def allreduce(x: np.ndarray, dtype: str, bits: int, group: int, bits2: int | None = None) -> dict:
    bits2 = bits if bits2 is None else bits2
    R, T, H = x.shape
    C = H // R
    g2 = min(group, C)
    v = widen(x, dtype).reshape(R, T, H // group, group)
    q1, s1, z1 = quantize(v, bits)
    xh = dequant(q1, s1, z1).reshape(R, T, H)
    y = xh[0].copy()
    for r in range(1, R):
        y = y + xh[r]
    q2, s2, z2 = quantize(y.reshape(T, H // g2, g2), bits2)
    o32 = dequant(q2, s2, z2).reshape(T, H)
    return dict(
        codes1=pack(q1.reshape(R * T, H), bits).reshape(R, T, -1), s1=s1, z1=z1,
        codes2=pack(q2.reshape(T, H), bits2), s2=s2, z2=z2, y=y, o32=o32,
        out=narrow(o32, dtype), group2=g2)

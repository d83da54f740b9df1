"""CPU oracle of the low-bit all-reduce codec (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it. The arithmetic lives in
`fc_oracle.c` (plain, single-threaded C built with -O2 -ffp-contract=off);
this module compiles it with gcc when needed and marshals numpy arrays.

Method: "Flash Communication: Reducing Tensor Parallelization Bottleneck for
Fast Large Language Model Inference" (TL;DR; Abstract; Figure 4; Figure 5,
right; Figure 3 for the transformer block around the all-reduce). Parity is
pinned by `tests/test_oracle_pins.py` (closed forms, error bounds, brute force,
integer arithmetic and library conversions); no function here is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = [
    "build", "lib", "F16", "BF16", "OracleError",
    "half_to_float", "float_to_half", "bf16_to_float", "float_to_bf16",
    "quantize_groups", "dequant_sum_requant", "dequantize", "quantize_f32",
    "allreduce", "stage2_group", "code_bytes", "sum_uncompressed", "dequantize_residual",
    "linear", "linear_quantize",
]

F16 = "f16"
BF16 = "bf16"
_DT = {F16: 0, BF16: 1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fc_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-frounding-math", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None

_ERRORS = {2: "shape", 3: "bits", 8: "out of range (non-finite, or fp16 scale/zero overflow)",
           9: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"oracle {where}: status {status} ({_ERRORS.get(status, '?')})")
        self.status = status


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (in-tree shared object)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_SO)
            P = ctypes.c_void_p
            I = ctypes.c_int
            L.ref_half_to_float.restype = ctypes.c_float
            L.ref_half_to_float.argtypes = [ctypes.c_uint16]
            L.ref_bf16_to_float.restype = ctypes.c_float
            L.ref_bf16_to_float.argtypes = [ctypes.c_uint16]
            L.ref_float_to_half.restype = ctypes.c_uint16
            L.ref_float_to_half.argtypes = [ctypes.c_float]
            L.ref_float_to_bf16.restype = ctypes.c_uint16
            L.ref_float_to_bf16.argtypes = [ctypes.c_float]
            L.ref_stage2_group.restype = I
            L.ref_stage2_group.argtypes = [I, I, I]
            L.ref_quantize_groups.restype = I
            L.ref_quantize_groups.argtypes = [P, I, I, I, I, I, I, P, P, P]
            L.ref_dequant_sum_requant.restype = I
            L.ref_dequant_sum_requant.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P]
            L.ref_dequant_sum_requant_mixed.restype = I
            L.ref_dequant_sum_requant_mixed.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P]
            L.ref_dequantize.restype = I
            L.ref_dequantize.argtypes = [P, P, P, I, I, I, I, I, P, P]
            L.ref_quantize_f32.restype = I
            L.ref_quantize_f32.argtypes = [P, ctypes.c_size_t, I, I, P, P, P]
            L.ref_sum_uncompressed.restype = I
            L.ref_sum_uncompressed.argtypes = [P, I, I, I, I, P]
            L.ref_dequantize_residual.restype = I
            L.ref_dequantize_residual.argtypes = [P, P, P, I, I, I, I, I, P, P]
            for name in ("ref_half_to_float_n", "ref_bf16_to_float_n",
                         "ref_float_to_half_n", "ref_float_to_bf16_n"):
                fn = getattr(L, name)
                fn.restype = None
                fn.argtypes = [P, P, ctypes.c_size_t]
            _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise OracleError(status, where)


# --- conversions ---

def _conv(name: str, src, src_dtype, dst_dtype) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(src, dtype=src_dtype))
    out = np.empty(a.shape, dtype=dst_dtype)
    getattr(lib(), name)(_p(a), _p(out), a.size)
    return out


def half_to_float(bits) -> np.ndarray:
    return _conv("ref_half_to_float_n", bits, np.uint16, np.float32)


def bf16_to_float(bits) -> np.ndarray:
    return _conv("ref_bf16_to_float_n", bits, np.uint16, np.float32)


def float_to_half(vals) -> np.ndarray:
    return _conv("ref_float_to_half_n", vals, np.float32, np.uint16)


def float_to_bf16(vals) -> np.ndarray:
    return _conv("ref_float_to_bf16_n", vals, np.float32, np.uint16)


# --- the method ---

def stage2_group(R: int, H: int, group: int) -> int:
    return lib().ref_stage2_group(R, H, group)


def code_bytes(n_elems: int, bits: int) -> int:
    return n_elems * bits // 8


def quantize_groups(x: np.ndarray, dtype: str, bits: int, group: int):
    """x: uint16 bit patterns [R, T, H] -> (codes1 [R, T, H*bits/8] u8, s1, z1 [R, T, H/group] u16)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, T, H = x.shape
    if H % group:
        raise OracleError(2, "quantize_groups")
    codes = np.zeros((R, T, code_bytes(H, bits)), dtype=np.uint8)
    s = np.zeros((R, T, H // group), dtype=np.uint16)
    z = np.zeros_like(s)
    _check(lib().ref_quantize_groups(_p(x), _DT[dtype], R, T, H, bits, group,
                                     _p(codes), _p(s), _p(z)), "quantize_groups")
    return codes, s, z


def dequant_sum_requant(codes1, s1, z1, R: int, T: int, H: int, bits: int, group: int,
                        want_y: bool = False, bits2: int | None = None):
    """Stage-1 payload -> (codes2 [T, H*bits2/8], s2, z2 [T, H/g2], y [T, H] f32 or None).
    `bits` is the stage-1 code width, `bits2` (default: the same) the stage-2 one."""
    bits2 = bits if bits2 is None else bits2
    g2 = stage2_group(R, H, group)
    if g2 <= 0 or H % g2:
        raise OracleError(2, "dequant_sum_requant")
    codes1 = np.ascontiguousarray(codes1, dtype=np.uint8)
    s1 = np.ascontiguousarray(s1, dtype=np.uint16)
    z1 = np.ascontiguousarray(z1, dtype=np.uint16)
    codes2 = np.zeros((T, code_bytes(H, bits2)), dtype=np.uint8)
    s2 = np.zeros((T, H // g2), dtype=np.uint16)
    z2 = np.zeros_like(s2)
    y = np.zeros((T, H), dtype=np.float32) if want_y else None
    _check(lib().ref_dequant_sum_requant_mixed(_p(codes1), _p(s1), _p(z1), R, T, H, bits, bits2,
                                               group, _p(codes2), _p(s2), _p(z2), _p(y)),
           "dequant_sum_requant")
    return codes2, s2, z2, y


def dequantize(codes2, s2, z2, T: int, H: int, bits: int, group2: int, dtype: str,
               want_o32: bool = False):
    """Stage-2 payload -> (out [T, H] uint16 bit patterns, o32 [T, H] f32 or None)."""
    codes2 = np.ascontiguousarray(codes2, dtype=np.uint8)
    s2 = np.ascontiguousarray(s2, dtype=np.uint16)
    z2 = np.ascontiguousarray(z2, dtype=np.uint16)
    out = np.zeros((T, H), dtype=np.uint16)
    o32 = np.zeros((T, H), dtype=np.float32) if want_o32 else None
    _check(lib().ref_dequantize(_p(codes2), _p(s2), _p(z2), T, H, bits, group2, _DT[dtype],
                                _p(out), _p(o32)), "dequantize")
    return out, o32


def quantize_f32(v: np.ndarray, bits: int, group: int):
    """Quantize flat binary32 values in groups (the stage-2 quantizer alone)."""
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    n = v.size
    codes = np.zeros(code_bytes(n, bits), dtype=np.uint8)
    s = np.zeros(n // group, dtype=np.uint16)
    z = np.zeros_like(s)
    _check(lib().ref_quantize_f32(_p(v), n, bits, group, _p(codes), _p(s), _p(z)), "quantize_f32")
    return codes, s, z


def allreduce(x: np.ndarray, dtype: str, bits: int, group: int, want_f32: bool = True,
              bits2: int | None = None) -> dict:
    """The whole path on one host: every intermediate of the emulated all-reduce.
    `bits` codes the reduce-scatter payload, `bits2` (default: the same) the all-gather one."""
    bits2 = bits if bits2 is None else bits2
    R, T, H = x.shape
    codes1, s1, z1 = quantize_groups(x, dtype, bits, group)
    codes2, s2, z2, y = dequant_sum_requant(codes1, s1, z1, R, T, H, bits, group, want_y=want_f32,
                                            bits2=bits2)
    g2 = stage2_group(R, H, group)
    out, o32 = dequantize(codes2, s2, z2, T, H, bits2, g2, dtype, want_o32=want_f32)
    return dict(codes1=codes1, s1=s1, z1=z1, codes2=codes2, s2=s2, z2=z2, y=y, o32=o32,
                out=out, group2=g2)


def sum_uncompressed(x: np.ndarray, dtype: str) -> np.ndarray:
    """The uncompressed all-reduce: out [T, H] = 16-bit rounding of the binary32 sum over r."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, T, H = x.shape
    out = np.zeros((T, H), dtype=np.uint16)
    _check(lib().ref_sum_uncompressed(_p(x), _DT[dtype], R, T, H, _p(out)), "sum_uncompressed")
    return out


def dequantize_residual(codes2, s2, z2, T: int, H: int, bits: int, group2: int, dtype: str,
                        residual: np.ndarray) -> np.ndarray:
    """Stage-2 payload and residual [T, H] 16-bit -> residual + all-reduce result, 16-bit."""
    codes2 = np.ascontiguousarray(codes2, dtype=np.uint8)
    s2 = np.ascontiguousarray(s2, dtype=np.uint16)
    z2 = np.ascontiguousarray(z2, dtype=np.uint16)
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    out = np.zeros((T, H), dtype=np.uint16)
    _check(lib().ref_dequantize_residual(_p(codes2), _p(s2), _p(z2), T, H, bits, group2,
                                         _DT[dtype], _p(residual), _p(out)), "dequantize_residual")
    return out


def linear(a: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """The row-parallel linear layer whose output each rank all-reduces (Figure 3:
    the attention output projection and the MLP down projection; Figure 5, left,
    names the two all-reduces o_proj and d_proj). Rank r holds its slice of the
    layer input, a[r] [T, K], and the matching input columns of the weight,
    w[r] [H, K] (a linear layer's [out, in] weight layout), and produces the
    partial sum y[r] = a[r] @ w[r]^T [T, H] in the activation dtype.

    Arithmetic: the dot products are taken in float64 (numpy's matmul, a library
    step), rounded to binary32 -- the value a binary32 accumulator holds when
    its accumulation is exact -- and then to the dtype, to nearest even.
      a [R, T, K], w [R, H, K] uint16 bit patterns -> y [R, T, H] uint16 bit patterns
    """
    widen = half_to_float if dtype == F16 else bf16_to_float
    narrow = float_to_half if dtype == F16 else float_to_bf16
    A = widen(np.ascontiguousarray(a, dtype=np.uint16)).astype(np.float64)
    W = widen(np.ascontiguousarray(w, dtype=np.uint16)).astype(np.float64)
    if A.ndim != 3 or W.ndim != 3 or A.shape[0] != W.shape[0] or A.shape[2] != W.shape[2]:
        raise OracleError(2, "linear")
    y64 = np.matmul(A, W.transpose(0, 2, 1))
    return narrow(y64.astype(np.float32))


def linear_quantize(a: np.ndarray, w: np.ndarray, dtype: str, bits: int, group: int) -> dict:
    """The linear layer followed by the quantization before the Reduce-Scatter
    (Figure 3's block with Figure 5's first quantization): y = linear(a, w), then
    the stage-1 codes of y exactly as quantize_groups gives them.
      -> dict(y [R, T, H], codes1 [R, T, H*bits/8], s1, z1 [R, T, H/group])"""
    y = linear(a, w, dtype)
    codes1, s1, z1 = quantize_groups(y, dtype, bits, group)
    return dict(y=y, codes1=codes1, s1=s1, z1=z1)

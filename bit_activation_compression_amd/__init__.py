"""Low-bit all-reduce activation codec for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI in `include/fc.h` (libfc.so, built from
`csrc/` by `build.py`). Every step of the codec runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with
torch on the input's device, and passes raw device pointers and the current
HIP stream. There is no fallback: if the library cannot be loaded, calls
raise.

Method: "Flash Communication: Reducing Tensor Parallelization Bottleneck for
Fast Large Language Model Inference" -- quantize the R partial sums before
the Reduce-Scatter, reduce and requantize each hidden chunk before the
All-Gather, dequantize after it (Figure 5, right; groups as in Figure 4).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "FcError", "lib", "library_path",
    "fc_quantize_groups", "fc_dequant_sum_requant", "fc_dequantize", "fc_allreduce_emulated",
    "fc_workspace_bytes", "fc_workspace_layout", "fc_stage2_group", "fc_status_string",
    "fc_sum_uncompressed", "fc_dequantize_residual", "fc_linear_quantize", "workspace_views",
    "fc_allreduce_emulated_noalloc", "NOALLOC_SCRATCH_BYTES",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libfc.so")

FC_F16, FC_BF16 = 0, 1
_DTYPES = {torch.float16: FC_F16, torch.bfloat16: FC_BF16}
EXPORTED_SYMBOLS = (
    "fc_quantize_groups", "fc_dequant_sum_requant", "fc_dequantize", "fc_allreduce_emulated",
    "fc_workspace_bytes", "fc_workspace_layout", "fc_stage2_group", "fc_status_string",
    "fc_sum_uncompressed", "fc_dequant_sum_requant_mixed", "fc_allreduce_emulated_mixed",
    "fc_workspace_bytes_mixed", "fc_workspace_layout_mixed",
    "fc_dequantize_residual", "fc_allreduce_emulated_residual", "fc_linear_quantize",
    "fc_allreduce_emulated_noalloc",
)
# FC_NOALLOC_SCRATCH_BYTES of include/fc.h: the payload scratch the library holds per device
NOALLOC_SCRATCH_BYTES = 64 << 20

_lock = threading.Lock()
_lib = None


class FcError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().fc_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfc.so (building it with hipcc first if it is absent)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                from . import build as _build
                _build.build()
            L = ctypes.CDLL(library_path)
            P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            L.fc_quantize_groups.argtypes = [P, I, I, I, I, I, I, P, P, P, P]
            L.fc_dequant_sum_requant.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P]
            L.fc_dequantize.argtypes = [P, P, P, I, I, I, I, I, P, P]
            L.fc_allreduce_emulated.argtypes = [P, I, I, I, I, I, I, P, P, Z, P]
            L.fc_sum_uncompressed.argtypes = [P, I, I, I, I, P, P]
            L.fc_dequant_sum_requant_mixed.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P]
            L.fc_allreduce_emulated_mixed.argtypes = [P, I, I, I, I, I, I, I, P, P, Z, P]
            L.fc_dequantize_residual.argtypes = [P, P, P, I, I, I, I, I, P, P, P]
            L.fc_allreduce_emulated_residual.argtypes = [P, I, I, I, I, I, I, I, P, P, P, Z, P]
            L.fc_linear_quantize.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P, P]
            L.fc_allreduce_emulated_noalloc.argtypes = [P, I, I, I, I, I, I, P, P]
            for f in (L.fc_linear_quantize, L.fc_quantize_groups, L.fc_dequant_sum_requant, L.fc_dequantize,
                      L.fc_allreduce_emulated, L.fc_sum_uncompressed,
                      L.fc_dequant_sum_requant_mixed, L.fc_allreduce_emulated_mixed,
                      L.fc_dequantize_residual, L.fc_allreduce_emulated_residual,
                      L.fc_allreduce_emulated_noalloc):
                f.restype = I
            L.fc_workspace_bytes_mixed.argtypes = [I, I, I, I, I, I]
            L.fc_workspace_bytes_mixed.restype = Z
            L.fc_workspace_layout_mixed.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Z),
                                                    ctypes.POINTER(Z)]
            L.fc_workspace_layout_mixed.restype = I
            L.fc_workspace_bytes.argtypes = [I, I, I, I, I]
            L.fc_workspace_bytes.restype = Z
            L.fc_workspace_layout.argtypes = [I, I, I, I, I, ctypes.POINTER(Z), ctypes.POINTER(Z)]
            L.fc_workspace_layout.restype = I
            L.fc_stage2_group.argtypes = [I, I, I]
            L.fc_stage2_group.restype = I
            L.fc_status_string.argtypes = [I]
            L.fc_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FcError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# torch's current stream as a raw handle without building a Stream object
# (a few microseconds per call, which matters for decode-sized calls); the
# public route where this accessor does not exist
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_current_stream is not None:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_current_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be float16 or bfloat16, not {t.dtype}")
    return _DTYPES[t.dtype]


def _room(t: torch.Tensor, name: str, nbytes: int, device) -> None:
    """A caller's buffer: a contiguous tensor on `device` of at least `nbytes`
    bytes (the library writes or reads that many through a raw pointer)."""
    _dev_tensor(t, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} needed")


def fc_status_string(status: int) -> str:
    return lib().fc_status_string(status).decode()


def fc_stage2_group(R: int, H: int, group: int) -> int:
    return lib().fc_stage2_group(R, H, group)


def fc_workspace_bytes(R: int, T: int, H: int, bits: int, group: int,
                       bits2: int | None = None) -> int:
    if bits2 is None or bits2 == bits:
        return lib().fc_workspace_bytes(R, T, H, bits, group)
    return lib().fc_workspace_bytes_mixed(R, T, H, bits, bits2, group)


def fc_workspace_layout(R: int, T: int, H: int, bits: int, group: int, bits2: int | None = None):
    """[(offset, size)] of the six workspace slices: codes1, s1, z1, codes2, s2, z2."""
    off = (ctypes.c_size_t * 6)()
    size = (ctypes.c_size_t * 6)()
    if bits2 is None or bits2 == bits:
        _check(lib().fc_workspace_layout(R, T, H, bits, group, off, size), "fc_workspace_layout")
    else:
        _check(lib().fc_workspace_layout_mixed(R, T, H, bits, bits2, group, off, size),
               "fc_workspace_layout_mixed")
    return [(off[i], size[i]) for i in range(6)]


def fc_quantize_groups(x: torch.Tensor, bits: int, group: int, codes1=None, s1=None, z1=None,
                       stream=None):
    """x [R, T, H] fp16/bf16 -> (codes1 [R, T, H*bits/8] u8, s1, z1 [R, T, H/group] fp16 bits)."""
    _dev_tensor(x, "x")
    R, T, H = x.shape
    dev = x.device
    if codes1 is None:
        codes1 = torch.empty((R, T, H * bits // 8), dtype=torch.uint8, device=dev)
    if s1 is None:
        s1 = torch.empty((R, T, max(H // group, 0)), dtype=torch.uint16, device=dev)
    if z1 is None:
        z1 = torch.empty_like(s1)
    _room(codes1, "codes1", R * T * H * bits // 8, dev)
    _room(s1, "s1", R * T * (H // group) * 2, dev)
    _room(z1, "z1", R * T * (H // group) * 2, dev)
    _check(lib().fc_quantize_groups(_ptr(x), _dt(x, "x"), R, T, H, bits, group, _ptr(codes1),
                                    _ptr(s1), _ptr(z1), _stream(stream, dev)), "fc_quantize_groups")
    return codes1, s1, z1


def fc_dequant_sum_requant(codes1, s1, z1, R: int, T: int, H: int, bits: int, group: int,
                           codes2=None, s2=None, z2=None, stream=None, bits2: int | None = None):
    """Stage-1 payload -> (codes2 [T, H*bits2/8], s2, z2 [T, H/g2]); bits2 defaults to bits."""
    bits2 = bits if bits2 is None else bits2
    for n, t in (("codes1", codes1), ("s1", s1), ("z1", z1)):
        _dev_tensor(t, n)
    dev = codes1.device
    g2 = fc_stage2_group(R, H, group)
    if codes2 is None:
        codes2 = torch.empty((T, H * bits2 // 8), dtype=torch.uint8, device=dev)
    if s2 is None:
        s2 = torch.empty((T, H // g2 if g2 else 0), dtype=torch.uint16, device=dev)
    if z2 is None:
        z2 = torch.empty_like(s2)
    _room(codes1, "codes1", R * T * H * bits // 8, dev)
    _room(s1, "s1", R * T * (H // group) * 2, dev)
    _room(z1, "z1", R * T * (H // group) * 2, dev)
    _room(codes2, "codes2", T * H * bits2 // 8, dev)
    _room(s2, "s2", T * (H // g2 if g2 else 0) * 2, dev)
    _room(z2, "z2", T * (H // g2 if g2 else 0) * 2, dev)
    if bits2 == bits:
        st = lib().fc_dequant_sum_requant(_ptr(codes1), _ptr(s1), _ptr(z1), R, T, H, bits, group,
                                          _ptr(codes2), _ptr(s2), _ptr(z2), _stream(stream, dev))
    else:
        st = lib().fc_dequant_sum_requant_mixed(_ptr(codes1), _ptr(s1), _ptr(z1), R, T, H, bits,
                                                bits2, group, _ptr(codes2), _ptr(s2), _ptr(z2),
                                                _stream(stream, dev))
    _check(st, "fc_dequant_sum_requant")
    return codes2, s2, z2


def fc_dequantize(codes2, s2, z2, T: int, H: int, bits: int, group2: int, dtype: torch.dtype,
                  out=None, stream=None):
    """Stage-2 payload -> out [T, H] of `dtype`."""
    for n, t in (("codes2", codes2), ("s2", s2), ("z2", z2)):
        _dev_tensor(t, n)
    dev = codes2.device
    if out is None:
        out = torch.empty((T, H), dtype=dtype, device=dev)
    _room(codes2, "codes2", T * H * bits // 8, dev)
    _room(s2, "s2", T * (H // group2 if group2 > 0 else 0) * 2, dev)
    _room(z2, "z2", T * (H // group2 if group2 > 0 else 0) * 2, dev)
    _room(out, "out", T * H * 2, dev)
    _check(lib().fc_dequantize(_ptr(codes2), _ptr(s2), _ptr(z2), T, H, bits, group2,
                               _dt(out, "out"), _ptr(out), _stream(stream, dev)), "fc_dequantize")
    return out


def fc_linear_quantize(a: torch.Tensor, w: torch.Tensor, bits: int, group: int, codes1=None,
                       s1=None, z1=None, y=None, stream=None):
    """Row-parallel linear layer of every rank with the stage-1 quantization in its
    epilogue: a [R, T, K], w [R, H, K] (fp16/bf16) -> (codes1, s1, z1, y) for the
    layer output y [R, T, H] = a @ w^T rounded to the dtype. y is written only when
    a tensor (or True, to allocate one) is passed; otherwise None is returned."""
    _dev_tensor(a, "a")
    _dev_tensor(w, "w")
    if a.dtype != w.dtype or a.dim() != 3 or w.dim() != 3 or a.shape[0] != w.shape[0] \
            or a.shape[2] != w.shape[2]:
        raise ValueError("a must be [R, T, K] and w [R, H, K] of one dtype")
    R, T, K = a.shape
    H = w.shape[1]
    dev = a.device
    if w.device != dev:
        raise ValueError(f"w is on {w.device}, a on {dev}")
    if codes1 is None:
        codes1 = torch.empty((R, T, H * bits // 8), dtype=torch.uint8, device=dev)
    if s1 is None:
        s1 = torch.empty((R, T, max(H // group, 0)), dtype=torch.uint16, device=dev)
    if z1 is None:
        z1 = torch.empty_like(s1)
    if y is True:
        y = torch.empty((R, T, H), dtype=a.dtype, device=dev)
    if y is not None and y.dtype != a.dtype:
        raise ValueError(f"y must have a's dtype ({a.dtype}), not {y.dtype}")
    _room(codes1, "codes1", R * T * H * bits // 8, dev)
    _room(s1, "s1", R * T * (H // group) * 2, dev)
    _room(z1, "z1", R * T * (H // group) * 2, dev)
    if y is not None:
        _room(y, "y", R * T * H * 2, dev)
    _check(lib().fc_linear_quantize(_ptr(a), _ptr(w), _dt(a, "a"), R, T, K, H, bits, group,
                                    _ptr(codes1), _ptr(s1), _ptr(z1), _ptr(y),
                                    _stream(stream, dev)), "fc_linear_quantize")
    return codes1, s1, z1, y


def fc_dequantize_residual(codes2, s2, z2, T: int, H: int, bits: int, group2: int,
                           residual: torch.Tensor, out=None, stream=None):
    """Stage-2 payload + residual [T, H] -> out [T, H] = residual + dequantized result
    (`out` may be `residual` itself for an in-place update)."""
    for n, t in (("codes2", codes2), ("s2", s2), ("z2", z2), ("residual", residual)):
        _dev_tensor(t, n)
    dev = codes2.device
    if out is None:
        out = torch.empty((T, H), dtype=residual.dtype, device=dev)
    if out.dtype != residual.dtype:
        raise ValueError("out and residual must have the same dtype")
    _room(codes2, "codes2", T * H * bits // 8, dev)
    _room(s2, "s2", T * (H // group2 if group2 > 0 else 0) * 2, dev)
    _room(z2, "z2", T * (H // group2 if group2 > 0 else 0) * 2, dev)
    _room(residual, "residual", T * H * 2, dev)
    _room(out, "out", T * H * 2, dev)
    _check(lib().fc_dequantize_residual(_ptr(codes2), _ptr(s2), _ptr(z2), T, H, bits, group2,
                                        _dt(residual, "residual"), _ptr(residual), _ptr(out),
                                        _stream(stream, dev)), "fc_dequantize_residual")
    return out


def fc_allreduce_emulated(x: torch.Tensor, bits: int, group: int, out=None, workspace=None,
                          stream=None, bits2: int | None = None, residual=None):
    """x [R, T, H] -> out [T, H]: the whole emulated all-reduce (three kernels).
    `bits` codes the reduce-scatter payload, `bits2` (default: the same) the all-gather one.
    With `residual` [T, H], out = residual + the all-reduce (the last kernel adds it)."""
    _dev_tensor(x, "x")
    bits2 = bits if bits2 is None else bits2
    R, T, H = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    if workspace is None:
        workspace = torch.empty(max(fc_workspace_bytes(R, T, H, bits, group, bits2), 1),
                                dtype=torch.uint8, device=dev)
    if out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    _room(out, "out", T * H * 2, dev)
    _room(workspace, "workspace", 0, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    if residual is not None:
        _room(residual, "residual", T * H * 2, dev)
        if residual.dtype != x.dtype or tuple(residual.shape) != (T, H):
            raise ValueError("residual must be [T, H] of x's dtype")
        st = lib().fc_allreduce_emulated_residual(_ptr(x), _dt(x, "x"), R, T, H, bits, bits2,
                                                  group, _ptr(residual), _ptr(out),
                                                  _ptr(workspace), ws_bytes, _stream(stream, dev))
    elif bits2 == bits:
        st = lib().fc_allreduce_emulated(_ptr(x), _dt(x, "x"), R, T, H, bits, group, _ptr(out),
                                         _ptr(workspace), ws_bytes, _stream(stream, dev))
    else:
        st = lib().fc_allreduce_emulated_mixed(_ptr(x), _dt(x, "x"), R, T, H, bits, bits2, group,
                                               _ptr(out), _ptr(workspace), ws_bytes,
                                               _stream(stream, dev))
    _check(st, "fc_allreduce_emulated")
    return out, workspace


def fc_allreduce_emulated_noalloc(x: torch.Tensor, bits: int, group: int, out=None,
                                  stream=None):
    """x [R, T, H] -> out [T, H]: fc_allreduce_emulated with both payloads in the library's
    own per-device scratch (the C call allocates nothing; pass `out` to allocate nothing
    here either). Raises FcError (FC_ERR_SCRATCH) when the payloads exceed
    NOALLOC_SCRATCH_BYTES. Calls that overlap in time on one device race on the scratch."""
    _dev_tensor(x, "x")
    R, T, H = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    if out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    _room(out, "out", T * H * 2, dev)
    _check(lib().fc_allreduce_emulated_noalloc(_ptr(x), _dt(x, "x"), R, T, H, bits, group,
                                               _ptr(out), _stream(stream, dev)),
           "fc_allreduce_emulated_noalloc")
    return out


def fc_sum_uncompressed(x: torch.Tensor, out=None, stream=None):
    """x [R, T, H] fp16/bf16 -> out [T, H]: the uncompressed all-reduce result (binary32 sum)."""
    _dev_tensor(x, "x")
    R, T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    _room(out, "out", T * H * 2, x.device)
    _check(lib().fc_sum_uncompressed(_ptr(x), _dt(x, "x"), R, T, H, _ptr(out),
                                     _stream(stream, x.device)), "fc_sum_uncompressed")
    return out


def workspace_views(workspace: torch.Tensor, R: int, T: int, H: int, bits: int, group: int,
                    bits2: int | None = None) -> dict:
    """Views of the payloads inside an fc_allreduce_emulated workspace."""
    bits2 = bits if bits2 is None else bits2
    lay = fc_workspace_layout(R, T, H, bits, group, bits2)
    g2 = fc_stage2_group(R, H, group)
    names = ("codes1", "s1", "z1", "codes2", "s2", "z2")
    shapes = ((R, T, H * bits // 8), (R, T, H // group), (R, T, H // group),
              (T, H * bits2 // 8), (T, H // g2), (T, H // g2))
    out = {}
    for name, (off, size), shape in zip(names, lay, shapes):
        raw = workspace[off:off + size]
        out[name] = raw.view(torch.uint16).view(shape) if name[0] in "sz" else raw.view(shape)
    return out

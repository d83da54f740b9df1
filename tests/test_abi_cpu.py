"""The C-ABI library without a GPU: it loads, exports every function that
include/fc.h declares, lays out the workspace as documented, and rejects
unsupported arguments before touching any device pointer (the pointers
passed here are fake, 16-byte aligned host integers; a validation bug would
surface as a HIP error, not as a write)."""
import ctypes
import os
import re

import pytest

import bit_activation_compression_amd as fc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fc.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced on the error paths
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared_functions(headers=(HEADER,)):
    src = "".join(open(h).read() for h in headers)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = fc.lib()
    names = _declared_functions()
    assert len(names) == 17
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(fc.EXPORTED_SYMBOLS)
    internal = sorted(set(_declared_functions(HEADERS)) - set(names))
    assert internal == ["fc_internal_clock_probe", "fc_internal_stream_probe"]
    for n in internal:
        assert hasattr(L, n), n


def test_no_kernel_launch_stub_left_undefined():
    """Every kernel's host-side launch stub is defined in the library (the
    host compiler pass can drop one silently; loading would then fail)."""
    import shutil
    import subprocess
    from bit_activation_compression_amd import build as libbuild
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    r = subprocess.run([nm, "-D", "--undefined-only", libbuild.LIB], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "__device_stub__" not in r.stdout


def test_status_strings():
    for s in range(9):
        assert fc.fc_status_string(s).startswith("FC_")
    assert "unknown" in fc.fc_status_string(99)


def test_stage2_group():
    assert fc.fc_stage2_group(4, 8192, 128) == 128
    assert fc.fc_stage2_group(4, 4096, 4096) == 1024
    assert fc.fc_stage2_group(2, 256, 128) == 128
    assert fc.fc_stage2_group(3, 4096, 128) == 0         # H % R != 0
    assert fc.fc_stage2_group(4, 4096, 96) == 0          # 96 does not divide 4096
    assert fc.fc_stage2_group(4, 4608, 96) == 96         # any even group dividing H
    assert fc.fc_stage2_group(3, 576, 96) == 96
    assert fc.fc_stage2_group(4, 6144, 6144) == 1536     # g > C: the chunk width
    assert fc.fc_stage2_group(2, 8, 2) == 2
    assert fc.fc_stage2_group(4, 36, 12) == 0            # g2 = C = 9 is odd
    assert fc.fc_stage2_group(2, 12, 3) == 0             # odd group
    assert fc.fc_stage2_group(4, 64, 64) == 16
    assert fc.fc_stage2_group(64, 512, 8) == 8
    assert fc.fc_stage2_group(128, 512, 8) == 4          # C = 4 < group: the chunk width
    assert fc.fc_stage2_group(128, 384, 8) == 0          # C = 3: odd


def test_workspace_layout_matches_payload_sizes():
    R, T, H, bits, g = 4, 8192, 8192, 4, 128
    lay = fc.fc_workspace_layout(R, T, H, bits, g)
    sizes = [s for _, s in lay]
    assert sizes == [R * T * H // 2, R * T * H // g * 2, R * T * H // g * 2,
                     T * H // 2, T * H // g * 2, T * H // g * 2]
    offs = [o for o, _ in lay]
    assert all(o % 256 == 0 for o in offs)
    assert all(offs[i] + sizes[i] <= offs[i + 1] for i in range(5))
    total = fc.fc_workspace_bytes(R, T, H, bits, g)
    assert total >= offs[5] + sizes[5] and total - (offs[5] + sizes[5]) < 256
    assert fc.fc_workspace_bytes(4, 8192, 8192, 5, 128) == 0
    lay48 = fc.fc_workspace_layout(R, T, H, 4, g, bits2=8)
    assert [s for _, s in lay48][0] == R * T * H // 2 and [s for _, s in lay48][3] == T * H
    lay84 = fc.fc_workspace_layout(R, T, H, 8, g, bits2=4)
    assert [s for _, s in lay84][0] == R * T * H and [s for _, s in lay84][3] == T * H // 2


def _q(*args):
    return fc.lib().fc_quantize_groups(*args)


@pytest.mark.parametrize("R,T,H,bits,g,status", [
    (4, 8, 512, 5, 128, 3),       # bits
    (4, 8, 512, 4, 96, 2),        # group does not divide H
    (4, 8, 510, 3, 3, 3),         # bits checked first
    (2, 8, 510, 4, 3, 2),         # odd group
    (2, 8, 512, 4, 0, 2),         # zero group
    (4, 8, 512, 4, 16384, 2),     # group above H
    (4, 8, 36, 4, 12, 2),         # stage-2 group (the chunk, 9) odd
    (4, 8, 512, 4, 1024, 2),      # group does not divide H
    (3, 8, 512, 4, 128, 2),       # H % R
    (0, 8, 512, 4, 128, 2),       # R
    (4, -1, 512, 4, 128, 2),      # T
    (128, 8, 384, 4, 8, 2),       # C = 3 gives an odd stage-2 group
])
def test_quantize_rejects_bad_shapes(R, T, H, bits, g, status):
    assert _q(FAKE, 0, R, T, H, bits, g, FAKE, FAKE, FAKE, None) == status


def test_pointer_checks_before_launch():
    assert _q(None, 0, 2, 8, 256, 8, 128, FAKE, FAKE, FAKE, None) == 1
    assert _q(FAKE, 0, 2, 8, 256, 8, 128, FAKE, None, FAKE, None) == 1
    assert _q(MISALIGNED, 0, 2, 8, 256, 8, 128, FAKE, FAKE, FAKE, None) == 4
    assert _q(FAKE, 0, 2, 8, 256, 8, 128, FAKE, FAKE, MISALIGNED, None) == 4
    assert _q(FAKE, 2, 2, 8, 256, 8, 128, FAKE, FAKE, FAKE, None) == 7   # dtype
    # T == 0: nothing to do, NULL pointers allowed
    assert _q(None, 0, 2, 0, 256, 8, 128, None, None, None, None) == 0


def test_other_entry_points_validate():
    L = fc.lib()
    assert L.fc_dequant_sum_requant(FAKE, FAKE, FAKE, 3, 8, 256, 4, 128, FAKE, FAKE, FAKE, None) == 2
    assert L.fc_dequant_sum_requant(FAKE, FAKE, None, 2, 8, 256, 4, 128, FAKE, FAKE, FAKE, None) == 1
    assert L.fc_dequantize(FAKE, FAKE, FAKE, 8, 256, 4, 96, 0, FAKE, None) == 2
    assert L.fc_dequantize(FAKE, FAKE, FAKE, 8, 256, 6, 128, 0, FAKE, None) == 3
    assert L.fc_dequantize(FAKE, FAKE, FAKE, 8, 256, 4, 128, 0, MISALIGNED, None) == 4
    need = fc.fc_workspace_bytes(2, 8, 256, 8, 128)
    assert L.fc_allreduce_emulated(FAKE, 0, 2, 8, 256, 8, 128, FAKE, FAKE, need - 1, None) == 5
    assert L.fc_allreduce_emulated(FAKE, 0, 2, 8, 256, 8, 128, None, FAKE, need, None) == 1
    assert L.fc_allreduce_emulated(None, 0, 2, 0, 256, 8, 128, None, None, 0, None) == 0
    assert L.fc_sum_uncompressed(FAKE, 0, 0, 8, 256, FAKE, None) == 2
    assert L.fc_sum_uncompressed(FAKE, 0, 2, 8, 250, FAKE, None) == 2
    assert L.fc_sum_uncompressed(FAKE, 3, 2, 8, 256, FAKE, None) == 7
    assert L.fc_sum_uncompressed(MISALIGNED, 0, 2, 8, 256, FAKE, None) == 4
    assert L.fc_sum_uncompressed(None, 0, 2, 0, 256, None, None) == 0
    # mixed widths
    assert L.fc_dequant_sum_requant_mixed(FAKE, FAKE, FAKE, 2, 8, 256, 4, 6, 128, FAKE, FAKE, FAKE, None) == 3
    assert L.fc_dequant_sum_requant_mixed(FAKE, FAKE, FAKE, 2, 8, 256, 5, 8, 128, FAKE, FAKE, FAKE, None) == 3
    need = fc.fc_workspace_bytes(2, 8, 256, 4, 128, bits2=8)
    assert L.fc_allreduce_emulated_mixed(FAKE, 0, 2, 8, 256, 4, 8, 128, FAKE, FAKE, need - 1, None) == 5
    assert L.fc_allreduce_emulated_mixed(None, 0, 2, 0, 256, 4, 8, 128, None, None, 0, None) == 0
    # the residual add folded into the last step
    assert L.fc_dequantize_residual(FAKE, FAKE, FAKE, 8, 256, 4, 96, 0, FAKE, FAKE, None) == 2
    assert L.fc_dequantize_residual(FAKE, FAKE, FAKE, 8, 256, 6, 128, 0, FAKE, FAKE, None) == 3
    assert L.fc_dequantize_residual(FAKE, FAKE, FAKE, 8, 256, 4, 128, 2, FAKE, FAKE, None) == 7
    assert L.fc_dequantize_residual(FAKE, FAKE, FAKE, 8, 256, 4, 128, 0, None, FAKE, None) == 1
    assert L.fc_dequantize_residual(FAKE, FAKE, FAKE, 8, 256, 4, 128, 0, MISALIGNED, FAKE,
                                    None) == 4
    assert L.fc_dequantize_residual(None, None, None, 0, 256, 4, 128, 0, None, None, None) == 0
    need = fc.fc_workspace_bytes(2, 8, 256, 4, 128)
    assert L.fc_allreduce_emulated_residual(FAKE, 0, 2, 8, 256, 4, 4, 128, None, FAKE, FAKE, need,
                                            None) == 1
    assert L.fc_allreduce_emulated_residual(FAKE, 0, 2, 8, 256, 4, 4, 128, MISALIGNED, FAKE, FAKE,
                                            need, None) == 4
    assert L.fc_allreduce_emulated_residual(FAKE, 0, 2, 8, 256, 4, 4, 128, FAKE, FAKE, FAKE,
                                            need - 1, None) == 5
    assert L.fc_allreduce_emulated_residual(FAKE, 0, 2, 8, 250, 4, 4, 128, FAKE, FAKE, FAKE, need,
                                            None) == 2
    assert L.fc_allreduce_emulated_residual(None, 0, 2, 0, 256, 4, 4, 128, None, None, None, 0,
                                            None) == 0
    # the linear layer with the stage-1 quantization in its epilogue
    LQ = L.fc_linear_quantize
    assert LQ(FAKE, FAKE, 1, 4, 8, 2000, 8192, 4, 128, FAKE, FAKE, FAKE, None, None) == 2  # K % 32
    assert LQ(FAKE, FAKE, 1, 4, 8, 2048, 8320, 4, 128, FAKE, FAKE, FAKE, None, None) == 2  # H % 256
    assert LQ(FAKE, FAKE, 1, 4, 8, 2048, 8192, 4, 512, FAKE, FAKE, FAKE, None, None) == 2  # group
    assert LQ(FAKE, FAKE, 1, 4, 8, 0, 8192, 4, 128, FAKE, FAKE, FAKE, None, None) == 2     # K = 0
    assert LQ(FAKE, FAKE, 1, 4, 8, (1 << 22) + 32, 8192, 4, 128, FAKE, FAKE, FAKE, None, None) == 2
    assert LQ(FAKE, FAKE, 1, 1, 8, 2048, (1 << 24) + 256, 4, 128, FAKE, FAKE, FAKE, None, None) == 2
    assert LQ(FAKE, FAKE, 1, 4, 8, 2048, 8192, 6, 128, FAKE, FAKE, FAKE, None, None) == 3
    assert LQ(FAKE, FAKE, 2, 4, 8, 2048, 8192, 4, 128, FAKE, FAKE, FAKE, None, None) == 7
    assert LQ(FAKE, None, 1, 4, 8, 2048, 8192, 4, 128, FAKE, FAKE, FAKE, None, None) == 1
    assert LQ(FAKE, FAKE, 1, 4, 8, 2048, 8192, 4, 128, FAKE, FAKE, FAKE, MISALIGNED, None) == 4
    assert LQ(None, None, 1, 4, 0, 2048, 8192, 4, 128, None, None, None, None, None) == 0


def test_noalloc_entry_point_validates_before_any_runtime_call():
    L = fc.lib()
    NA = L.fc_allreduce_emulated_noalloc
    assert NA(FAKE, 0, 3, 8, 256, 4, 128, FAKE, None) == 2          # H % R
    assert NA(FAKE, 0, 2, 8, 256, 4, 96, FAKE, None) == 2           # group
    assert NA(FAKE, 0, 2, 8, 256, 6, 128, FAKE, None) == 3          # bits
    assert NA(FAKE, 2, 2, 8, 256, 4, 128, FAKE, None) == 7          # dtype
    assert NA(FAKE, 0, 2, 8, 256, 4, 128, None, None) == 1
    assert NA(MISALIGNED, 0, 2, 8, 256, 4, 128, FAKE, None) == 4
    assert NA(None, 0, 2, 0, 256, 4, 128, None, None) == 0          # T == 0
    # payloads larger than the library's fixed scratch: rejected, nothing enqueued
    assert fc.fc_workspace_bytes(4, 8192, 8192, 4, 128) > fc.NOALLOC_SCRATCH_BYTES
    assert NA(FAKE, 1, 4, 8192, 8192, 4, 128, FAKE, None) == 8


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define FC_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fc.NOALLOC_SCRATCH_BYTES


def test_stream_probe_validates():
    L = fc.lib()
    P = L.fc_internal_stream_probe
    P.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    assert P(4, 4, FAKE, FAKE, 1024, None) == 2
    assert P(-1, 4, FAKE, FAKE, 1024, None) == 2
    assert P(3, 5, FAKE, FAKE, 1024, None) == 2
    assert P(3, 4, FAKE, MISALIGNED, 1024, None) == 4
    assert P(0, 3, FAKE, FAKE, 1024, None) == 2
    assert P(0, 16, FAKE, FAKE, 1024, None) == 2
    assert P(0, 4, None, FAKE, 1024, None) == 1
    assert P(0, 4, MISALIGNED, FAKE, 1024, None) == 4
    assert P(0, 4, FAKE, FAKE, 1000, None) == 4
    assert P(0, 4, None, None, 0, None) == 0


def test_clock_probe_validates():
    L = fc.lib()
    P = L.fc_internal_clock_probe
    P.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert P(None, 100, None) == 1
    assert P(FAKE, 0, None) == 2
    assert P(FAKE, (1 << 20) + 1, None) == 2
    assert P(ctypes.c_void_p(0x10004), 100, None) == 4

"""The Python binding's own checks (GPU tensors needed): caller buffers are
size-, device-, dtype- and layout-checked before a raw pointer reaches the
library, and the library's status codes surface as FcError.
"""
from __future__ import annotations

import pytest
import torch

import bit_activation_compression_amd as fc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    fc.lib()
    yield


def _x(R=2, T=8, H=256, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda").manual_seed(3)
    return torch.randn((R, T, H), generator=g, device="cuda").to(dtype)


def test_short_output_buffers_are_refused():
    x = _x()
    with pytest.raises(ValueError, match="codes1 holds"):
        fc.fc_quantize_groups(x, 4, 128, codes1=torch.empty(2 * 8 * 128 - 1, dtype=torch.uint8,
                                                             device="cuda"))
    with pytest.raises(ValueError, match="s1 holds"):
        fc.fc_quantize_groups(x, 4, 128, s1=torch.empty(2 * 8 * 2 - 1, dtype=torch.uint16,
                                                         device="cuda"))
    c1, s1, z1 = fc.fc_quantize_groups(x, 4, 128)
    with pytest.raises(ValueError, match="codes2 holds"):
        fc.fc_dequant_sum_requant(c1, s1, z1, 2, 8, 256, 4, 128,
                                  codes2=torch.empty(10, dtype=torch.uint8, device="cuda"))
    c2, s2, z2 = fc.fc_dequant_sum_requant(c1, s1, z1, 2, 8, 256, 4, 128)
    with pytest.raises(ValueError, match="out holds"):
        fc.fc_dequantize(c2, s2, z2, 8, 256, 4, 128, torch.bfloat16,
                         out=torch.empty((8, 255), dtype=torch.bfloat16, device="cuda"))
    # inputs too short for the stated shape
    with pytest.raises(ValueError, match="codes1 holds"):
        fc.fc_dequant_sum_requant(c1[:1], s1, z1, 2, 8, 256, 4, 128)
    with pytest.raises(ValueError, match="out holds"):
        fc.fc_allreduce_emulated(x, 4, 128, out=torch.empty((8, 128), dtype=x.dtype, device="cuda"))
    with pytest.raises(ValueError, match="y holds"):
        a = _x(2, 8, 64)
        w = _x(2, 256, 64)
        fc.fc_linear_quantize(a, w, 4, 128, y=torch.empty((2, 8, 255), dtype=a.dtype, device="cuda"))


def test_layout_dtype_and_device_are_checked():
    x = _x()
    with pytest.raises(ValueError, match="contiguous"):
        fc.fc_sum_uncompressed(x, out=torch.empty((256, 8), dtype=x.dtype, device="cuda").t())
    with pytest.raises(ValueError, match="float16 or bfloat16"):
        fc.fc_quantize_groups(x.float(), 4, 128)
    with pytest.raises(ValueError, match="x's dtype"):
        fc.fc_allreduce_emulated(x, 4, 128, out=torch.empty((8, 256), dtype=torch.float16,
                                                             device="cuda"))
    with pytest.raises(ValueError, match="GPU tensor"):
        fc.fc_sum_uncompressed(x, out=torch.empty((8, 256), dtype=x.dtype))
    # the residual is a caller buffer like the others, and it must be [T, H]
    with pytest.raises(ValueError, match="GPU tensor"):
        fc.fc_allreduce_emulated(x, 4, 128, residual=torch.empty((8, 256), dtype=x.dtype))
    with pytest.raises(ValueError, match="residual holds"):
        fc.fc_allreduce_emulated(x, 4, 128, residual=torch.empty((8, 255), dtype=x.dtype,
                                                                  device="cuda"))
    with pytest.raises(ValueError, match=r"residual must be \[T, H\]"):
        fc.fc_allreduce_emulated(x, 4, 128, residual=torch.empty((4, 512), dtype=x.dtype,
                                                                  device="cuda"))
    # the layer output must have the operands' dtype (a float32 buffer of the same
    # byte count would otherwise receive 16-bit values)
    a = _x(2, 8, 64)
    w = _x(2, 256, 64)
    with pytest.raises(ValueError, match="y must have a's dtype"):
        fc.fc_linear_quantize(a, w, 4, 128, y=torch.empty((2, 8, 128), dtype=torch.float32,
                                                          device="cuda"))


def test_library_status_becomes_fc_error():
    x = _x()
    with pytest.raises(fc.FcError) as e:
        fc.fc_quantize_groups(x, 6, 128)
    assert e.value.status == 3            # FC_ERR_BITS
    with pytest.raises(fc.FcError) as e:
        fc.fc_quantize_groups(x, 4, 96)   # not a power of two
    assert e.value.status == 2            # FC_ERR_SHAPE
    need = fc.fc_workspace_bytes(2, 8, 256, 4, 128)
    with pytest.raises(fc.FcError) as e:
        fc.fc_allreduce_emulated(x, 4, 128, workspace=torch.empty(need - 1, dtype=torch.uint8,
                                                                   device="cuda"))
    assert e.value.status == 5            # FC_ERR_WORKSPACE


def test_workspace_of_any_element_type_counts_bytes():
    """A workspace tensor of 4-byte elements is measured in bytes, not elements."""
    x = _x()
    ref, _ = fc.fc_allreduce_emulated(x, 4, 128)
    need = fc.fc_workspace_bytes(2, 8, 256, 4, 128)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
    out, _ = fc.fc_allreduce_emulated(x, 4, 128, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

"""Instruction-level guard on the gfx950 code the kernels compile to.

The codec is specified step by step in binary32 with round-half-to-even
(asymmetric min/max quantizer of "Flash Communication: Reducing Tensor
Parallelization Bottleneck for Fast Large Language Model Inference",
Figures 4 and 5). Some instructions the compiler may pick would change that
rounding without changing the source:
  - v_fma_mix{lo,hi}_f16 / v_mad_mix{lo,hi}_f16: an fma fused with the
    following fp32 -> fp16 conversion rounds once instead of twice;
  - v_cvt_pkrtz_f16_f32: rounds toward zero;
  - v_pk_{fma,mul,add}_f32: packed fp32 forms the build flags keep out;
and scratch traffic would mean register spills on the hot path.
This compiles every kernel source to device assembly with the build's own
flags and checks that none of them appear.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from bit_activation_compression_amd import build as libbuild

FORBIDDEN = re.compile(r"^\s+(v_fma_mix(lo|hi)_f16|v_mad_mix(lo|hi)_f16|v_cvt_pkrtz_f16_f32|"
                       r"v_pk_fma_f32|v_pk_mul_f32|v_pk_add_f32|scratch_(load|store)\w*)\b", re.M)
KERNEL_SOURCES = [s for s in libbuild.SOURCES if s != "fc_api.hip"]


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [libbuild.HIPCC, *libbuild.FLAGS, "--cuda-device-only", "-S",
           os.path.join(libbuild.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(libbuild.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
            asm = dict(zip(KERNEL_SOURCES, ex.map(lambda s: _device_asm(s, d), KERNEL_SOURCES)))
    return asm


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_rounding_changing_or_spilling_instructions(device_asm, src):
    bad = sorted({m.group(1) for m in FORBIDDEN.finditer(device_asm[src])})
    assert not bad, f"{src}: {bad}"


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_private_segment(device_asm, src):
    sizes = [int(v) for v in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", device_asm[src])]
    assert sizes and max(sizes) == 0


def test_kernels_preserve_denormals(device_asm):
    for src, asm in device_asm.items():
        assert set(re.findall(r"\.amdhsa_float_denorm_mode_32 (\d+)", asm)) == {"3"}, src
        assert set(re.findall(r"\.amdhsa_float_denorm_mode_16_64 (\d+)", asm)) == {"3"}, src

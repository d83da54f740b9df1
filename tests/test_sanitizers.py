"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The CPU oracle (oracle/fc_oracle.c) linked into a small driver
   (tests/sanitize/oracle_driver.c) built with -fsanitize=address,undefined:
   every entry point runs on workload-shaped and edge-value cases, with
   exactly-sized buffers; the run must be free of sanitizer reports, and its
   outputs must equal, byte for byte, those of the normal oracle build the
   other tests use.
2. The C ABI's host-side argument checks and workspace layout
   (csrc/fc_validate.h, the code fc_api.hip compiles) in a driver
   (tests/sanitize/validate_driver.cpp) built the same way, over a grid of
   arguments; its answers must equal libfc.so's for the same arguments.
"""
import ctypes
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build(cc, srcs, out, extra):
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not available")
    r = subprocess.run([cc, *SAN, *extra, *srcs, "-o", out, "-lm"], capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("sanitizer runtime not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, env=ENV, timeout=300, **kw)
    err = r.stderr.decode(errors="replace")
    assert "AddressSanitizer" not in err and "runtime error" not in err and \
        "LeakSanitizer" not in err, err[-3000:]
    assert r.returncode == 0, err[-3000:]
    return r.stdout


def _edge_operands(R, T, H, dtype):
    """Constant groups, signed zeros, subnormals and large magnitudes, fp16 or bf16."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((R, T, H)).astype(np.float32)
    v[:, 0, :] = 3.0                                # constant rows
    v[:, 1, ::2] = -0.0
    v[:, 1, 1::2] = 0.0
    v[:, 2, :] = rng.standard_normal(H).astype(np.float32) * 1e-6   # fp16 subnormal range
    v[:, 3, :] = rng.standard_normal(H).astype(np.float32) * 3000.0
    return synth.operands_from_values(v, dtype)


CASES = [  # (label, R, T, H, dtype, bits1, bits2, group, source)
    ("tiny", 2, 8, 256, "f16", 8, 8, 128, "tiny"),
    ("decode-like", 8, 4, 1024, "bf16", 4, 4, 128, "decode"),
    ("group over chunks", 4, 4, 4096, "f16", 4, 4, 4096, "sweep_int4_g4096"),
    ("mixed widths", 4, 3, 512, "bf16", 4, 8, 64, "llama3_70b_prefill"),
    ("groups of 96, R = 3", 3, 5, 576, "f16", 8, 4, 96, "llama3_8b_prefill"),
    ("groups of 2", 2, 2, 8, "f16", 4, 4, 2, "tiny"),
    ("edge values f16", 2, 4, 256, "f16", 4, 4, 32, None),
    ("edge values bf16", 4, 4, 512, "bf16", 8, 4, 16, None),
    ("no tokens", 2, 0, 256, "f16", 4, 4, 128, "tiny"),
]


def _operands(case):
    label, R, T, H, dt, b1, b2, g, src = case
    if src is None:
        return _edge_operands(R, T, H, dt)
    w = synth.workload(src).with_(R=R, T=T, H=H, dtype=dt, bits=b1, group=g)
    return synth.operands(w, 11)


def test_oracle_under_sanitizers_matches_normal_build(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build("gcc", [os.path.join(ROOT, "oracle", "fc_oracle.c"),
                   os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")], exe,
           ["-std=c11", "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
            "-fexcess-precision=standard"])
    blob = [struct.pack("<i", len(CASES))]
    expect = []
    for case in CASES:
        label, R, T, H, dt, b1, b2, g, _ = case
        x = _operands(case)
        rng = np.random.default_rng(7)
        res = synth.operands_from_values(rng.standard_normal((T, H)).astype(np.float32) * 2, dt)
        blob.append(struct.pack("<7i", R, T, H, 0 if dt == "f16" else 1, b1, b2, g))
        blob.append(np.ascontiguousarray(x, dtype=np.uint16).tobytes())
        blob.append(np.ascontiguousarray(res, dtype=np.uint16).tobytes())
        # the normal build, through the package the other tests use
        c1, s1, z1 = oracle.quantize_groups(x, dt, b1, g)
        c2, s2, z2, y = oracle.dequant_sum_requant(c1, s1, z1, R, T, H, b1, g, want_y=True, bits2=b2)
        g2 = oracle.stage2_group(R, H, g)
        out, o32 = oracle.dequantize(c2, s2, z2, T, H, b2, g2, dt, want_o32=True)
        ro = oracle.dequantize_residual(c2, s2, z2, T, H, b2, g2, dt, res)
        su = oracle.sum_uncompressed(x, dt)
        c3, s3, z3 = oracle.quantize_f32(y, b2, g2)
        parts = [struct.pack("<6i", 0, 0, 0, 0, 0, 0), c1, s1, z1, c2, s2, z2,
                 np.asarray(y, np.float32), out, np.asarray(o32, np.float32), ro, su, c3, s3, z3]
        expect.append(b"".join(p if isinstance(p, bytes) else np.ascontiguousarray(p).tobytes()
                               for p in parts))
    expect.append(struct.pack("<5i", 3, 2, 2, 2, 2))
    cases = tmp_path / "cases.bin"
    cases.write_bytes(b"".join(blob))
    got_file = tmp_path / "out.bin"
    _run([exe, str(cases), str(got_file)])
    got = got_file.read_bytes()
    want = b"".join(expect)
    assert len(got) == len(want)
    pos = 0
    for case, part in zip(CASES + [("argument errors",)], expect):
        assert got[pos:pos + len(part)] == part, case[0]
        pos += len(part)


def test_abi_validation_under_sanitizers_matches_library(tmp_path):
    import bit_activation_compression_amd as fc
    exe = str(tmp_path / "validate_driver")
    csrc = os.path.join(ROOT, "bit_activation_compression_amd", "csrc")
    _build("g++", [os.path.join(ROOT, "tests", "sanitize", "validate_driver.cpp")], exe,
           ["-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}"])
    lines = _run([exe]).decode().splitlines()
    L = fc.lib()
    Z = ctypes.c_size_t
    n_ok = 0
    for line in lines[:-1]:
        args, res = line.split(" : ")
        R, T, H, b1, b2, g = (int(v) for v in args.split())
        vals = [int(v) for v in res.split()]
        off, size = (Z * 6)(), (Z * 6)()
        st = L.fc_workspace_layout_mixed(R, T, H, b1, b2, g, off, size)
        assert st == vals[0], line
        if st == 0:
            n_ok += 1
            g2, total = vals[1], vals[2]
            assert fc.fc_workspace_bytes(R, T, H, b1, g, bits2=b2) == total, line
            assert [x for i in range(6) for x in (off[i], size[i])] == vals[3:], line
            assert fc.fc_stage2_group(R, H, g) == g2, line
    assert n_ok > 1000
    assert lines[-1] == "ptrs 0 1 4 0"

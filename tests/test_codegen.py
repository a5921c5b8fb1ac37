"""Checks on the gfx950 code the kernels compile to (our own code objects).

A matrix-core instruction writes its result registers while later passes
still read the A/B sources, so a destination that overlaps A or B silently
corrupts the result (seen on rows 4k+2, 4k+3 of a 16x16 step).  The kernels
guard every matrix-core call against it; this test compiles each kernel source
to device assembly and verifies that no MFMA destination overlaps its A or B
operand (the accumulator input may equal the destination).

Every build disables packed fp32 instructions for the device code; a second
check verifies that none of the three packed fp32 arithmetic instructions
appears in the kernels' assembly.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b")


def _regs(tok):
    m = _REG.fullmatch(tok.strip())
    if not m:
        return None
    if m.group(1):
        return (m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1)))
    return (m.group(4), {int(m.group(5))})


def _device_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--offload-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


_ASMS = None


def _all_asm():
    global _ASMS
    if _ASMS is None:
        srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
        with tempfile.TemporaryDirectory() as td, cf.ThreadPoolExecutor(4) as ex:
            _ASMS = (srcs, list(ex.map(lambda s: _device_asm(s, td), srcs)))
    return _ASMS


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_packed_fp32_arithmetic():
    srcs, asms = _all_asm()
    bad = []
    for src, asm in zip(srcs, asms):
        for line in asm.splitlines():
            op = line.strip().split(None, 1)[0] if line.strip() else ""
            if op in ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"):
                bad.append(f"{os.path.basename(src)}: {line.strip()}")
    assert not bad, bad[:10]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_mfma_destination_overlaps_sources():
    srcs, asms = _all_asm()
    bad, n = [], 0
    for src, asm in zip(srcs, asms):
        for line in asm.splitlines():
            line = line.strip()
            if not line.startswith("v_mfma"):
                continue
            ops = [o for o in line.split(None, 1)[1].split(",")]
            d, a, b = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
            n += 1
            for s in (a, b):
                if d and s and d[0] == s[0] and d[1] & s[1]:
                    bad.append(f"{os.path.basename(src)}: {line}")
    assert n > 50, "no matrix-core instructions found"
    assert not bad, bad[:10]

"""Checks on the generated gfx950 code of libtaco (CPU: hipcc cross-compiles
the device code here; nothing runs on a GPU).

* m0 is written only by the direct-to-LDS copies' inline assembly.  clang
  warns that it may not honour an m0 clobber, so the compiler itself must use
  m0 nowhere in the library.
* No kernel calls a function: every helper and lambda is inlined (a lambda
  left out of line is reached through s_swappc with its captures in
  scratch memory).
* The fused kernels spill no VGPRs.  They wait for their LDS copies by count
  (loads complete in issue order); scratch spills are vector memory
  operations of their own, which would only make those waits longer, but a
  spilled value reloaded while copies are in flight stalls behind them.
"""
import os
import re
import subprocess

import pytest

from fp8_compression_tensor_taco_amd import build


@pytest.fixture(scope="module")
def device_code(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "taco.s")
    res = subprocess.run([hipcc, *build.compile_flags(), "--cuda-device-only", "-S", *build.SOURCES,
                          "-o", out, "-Rpass-analysis=kernel-resource-usage"],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read(), res.stderr


def test_m0_is_only_written_by_the_copy_asm(device_code):
    asm, _ = device_code
    inside = False
    outside = []
    for line in asm.splitlines():
        if "ASMSTART" in line:
            inside = True
            continue
        if "ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0]
        if not inside and re.search(r"\bm0\b", code):
            outside.append(line.strip())
    assert not outside, outside[:5]
    assert asm.count("global_load_lds_dwordx4") > 0      # the copies are there


def test_fused_kernels_do_not_spill(device_code):
    _, remarks = device_code
    name, spills = None, {}
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"VGPRs Spill: (\d+)", line)
        if m and name and re.search(r"compress_fused_(lds|ring)_kernel|decompress_sum_compress_kernel", name):
            spills[name] = int(m.group(1))
    assert len(spills) >= 10, sorted(spills)
    assert all(v == 0 for v in spills.values()), {k: v for k, v in spills.items() if v}


def test_no_kernel_calls_a_function(device_code):
    asm, _ = device_code
    assert "s_swappc_b64" not in asm
    assert "s_setpc_b64" not in asm

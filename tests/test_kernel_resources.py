"""Every libdsa kernel compiles for gfx950 without VGPR spills.

A spilled VGPR lives in scratch memory, and its reload inside a tile loop
needs vmcnt(0) -- which also waits for every direct global->LDS copy the
kernel has in flight (the copies are counted by the same counter), turning a
prefetch pipeline into a stall.  The kernels sit close to the 256-VGPR limit
of two waves per SIMD, so a small source change can tip one over; this test
reads the compiler's resource remarks (CPU only: hipcc cross-compiles).
"""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

from sparse_attention_fp8_amd import build

SOURCES = sorted(glob.glob(os.path.join(build.CSRC, "*.hip")))


def _have_hipcc():
    try:
        return os.path.exists(build.hipcc())
    except RuntimeError:
        return False


def _resource_remarks(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [build.hipcc(), "-x", "hip", "-c", src, "-o", obj, "--cuda-device-only",
           "-Rpass-analysis=kernel-resource-usage"] + build.common_flags()
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"VGPRs Spill: (\d+)", line)
        if m and name:
            kernels[name] = int(m.group(1))
    return src, kernels


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_no_kernel_spills_vgprs(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _resource_remarks(s, str(tmp_path)), SOURCES))
    seen = 0
    spilled = []
    for src, kernels in results:
        seen += len(kernels)
        spilled += [(os.path.basename(src), k, n) for k, n in kernels.items() if n > 0]
    assert seen >= 10, f"expected the resource remarks of every kernel, parsed {seen}"
    assert not spilled, f"kernels spilling VGPRs to scratch: {spilled}"

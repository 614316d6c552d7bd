"""Every gfx950 kernel compiles without register spills or scratch memory.

Each HIP source is compiled for the device only, with the library's own flags, under the
compiler's kernel resource-usage remarks; a kernel that spills VGPRs or SGPRs or needs
per-lane scratch fails.  (Spills crept in once when two epilogues of one kernel were
each fine alone; they cost the prefill GEMM ~4 % and the int8 GEMM ~12 %.)  No GPU is
needed: hipcc cross-compiles.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from w4a16_gemm_amd import build

HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _usage(src):
    cmd = [build.HIPCC, *build.COMMON, *build.EXTRA.get(src, []), "--cuda-device-only", "-c",
           "-Rpass-analysis=kernel-resource-usage", os.path.join(build.CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    kernels, cur = {}, None
    for line in r.stdout.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_no_spills_or_scratch():
    with cf.ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        usage = dict(zip(HIP_SOURCES, ex.map(_usage, HIP_SOURCES)))
    bad = []
    n = 0
    for src, kernels in usage.items():
        for name, u in kernels.items():
            n += 1
            assert set(u) == {"ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill"}, (src, name, u)
            if any(v != 0 for v in u.values()):
                bad.append((src, name, u))
    assert n >= 40, usage  # every template instance reported
    assert not bad, bad

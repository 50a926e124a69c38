"""Every HIP kernel compiles for gfx950 without private (scratch) memory or VGPR
spills (an SGPR spill with no scratch is kept in a VGPR lane).  A kernel that silently falls back to scratch (an array the compiler could not
keep in registers) runs several times slower, so this is checked on the CPU at build
time from the compiler's own resource report."""
import concurrent.futures
import os
import re
import subprocess

import pytest

from draft_kv_attention_amd import build as B


def _resources(src):
    cmd = [B.HIPCC, *B.COMMON_FLAGS, "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and cur:
            out[cur][m.group(1)] = int(m.group(2))
    return src, out


@pytest.fixture(scope="module")
def report():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(_resources, B.sources()))


def test_no_scratch_no_spills(report):
    kernels = 0
    for src, ks in report.items():
        for name, res in ks.items():
            kernels += 1
            assert res.get("ScratchSize [bytes/lane]", 0) == 0, (src, name, res)
            # SGPR spills without scratch live in VGPR lanes (v_writelane), no memory.
            assert res.get("VGPRs Spill", 0) == 0, (src, name, res)
    assert kernels >= 20

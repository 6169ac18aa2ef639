"""Every kernel of libengram keeps its registers in registers: no private
(scratch) memory per lane and no vector-register spills (scalar registers
that spill into lanes of vector registers touch no memory and are allowed).  A register budget tightened with an
occupancy attribute once made the compiler spill inside the backward's tile
kernel, and those builds gave wrong sums on the GPU; this check catches any
kernel that starts spilling, on the CPU, from the compiler's resource report."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from hashed_gram_embedding_engram_amd import build as B


def resource_report(src):
    cmd = [B.HIPCC] + B.COMMON_FLAGS + ["-c", "-x", "hip", os.path.join(B.CSRC, src), "-o", os.devnull,
                                        "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return src, kernels


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc is missing")
def test_no_kernel_uses_scratch():
    srcs = [s for s in B.SOURCES + B.PROBE_SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        reports = list(ex.map(resource_report, srcs))
    seen = 0
    for src, kernels in reports:
        for name, r in kernels.items():
            seen += 1
            assert r.get("ScratchSize [bytes/lane]", 0) == 0, (src, name, r)
            assert r.get("VGPRs Spill", 0) == 0, (src, name, r)
    assert seen >= 20

"""Every kernel variant keeps its state in registers and LDS: the compiler's
resource-usage report must show no scratch (private per-lane memory) for any
instantiated kernel. Scratch would mean spilled state going to device memory
on every use, against the premise of the method (LRAgent: Efficient KV Cache
Sharing for Multi-LoRA LLM Agents, abstract: the adapter part is rebuilt on
the fly rather than materialised).

The translation units are compiled for the device only, with the library's
own flags, so the variants checked are exactly the ones the library holds.
Runs on the CPU (hipcc cross-compiles for gfx950)."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from shared_base_kv_amd import build as B

HIPCC = B.HIPCC
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")

KERNEL_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def _report(src):
    cmd = [HIPCC, *B.FLAGS, "--cuda-device-only", "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            kernels[name] = int(m.group(1))
            name = None
    return src, kernels


@pytest.fixture(scope="module")
def reports():
    with cf.ThreadPoolExecutor(max_workers=min(8, len(KERNEL_SOURCES))) as ex:
        return dict(ex.map(_report, KERNEL_SOURCES))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_uses_scratch(reports, src):
    kernels = reports[src]
    assert kernels, f"no kernel found in the resource report of {src}"
    spills = {k: v for k, v in kernels.items() if v}
    assert not spills, f"{src}: kernels with scratch (bytes/lane): {spills}"

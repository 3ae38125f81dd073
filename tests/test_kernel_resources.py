"""Every HIP kernel of the library compiles for gfx950 without scratch memory
(no register spills, no private arrays): the compiler's resource-usage
remarks, per kernel, for each source file. CPU only (cross-compiles)."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from long_context_fine_amd import build

SOURCES = sorted(f for f in os.listdir(build.CSRC) if f.endswith(".hip"))


def _usage(src):
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [build._hipcc(), *build._flags(), "-x", "hip", "-c", os.path.join(build.CSRC, src),
               "--cuda-device-only", "-o", os.path.join(tmp, "k.o"),
               "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and cur:
            kernels[cur] = int(m.group(1))
    return src, kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_kernel_uses_scratch():
    with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        results = dict(ex.map(_usage, SOURCES))
    seen = 0
    for src, kernels in results.items():
        assert kernels, f"{src}: no resource-usage remarks"
        seen += len(kernels)
        spilled = {k: v for k, v in kernels.items() if v}
        assert not spilled, f"{src}: scratch bytes per lane {spilled}"
    assert seen >= 40

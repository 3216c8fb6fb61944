"""No kernel of the library spills registers to scratch memory: each source is
compiled for gfx950 (device code only, the library's flags) with the compiler's
resource-usage report, and every kernel must report a scratch size of 0."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_gqa_index_amd import build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="no hipcc")


def _report(src, tmp):
    cmd = build.hipcc_command(os.path.join(tmp, os.path.basename(src) + ".o"), sources=[src])
    cmd = [c for c in cmd if c not in ("-shared",)] + ["-c", "--cuda-device-only",
                                                         "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = {}
    for block in re.split(r"remark: Function Name: ", r.stderr)[1:]:
        name = block.split()[0]
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        out[name] = int(m.group(1))
    return out


def test_no_kernel_spills(tmp_path):
    with ThreadPoolExecutor(len(build.SOURCES)) as ex:
        reports = list(ex.map(lambda s: _report(s, str(tmp_path)), build.SOURCES))
    kernels = {k: v for r in reports for k, v in r.items()}
    assert len(kernels) > 50  # every instantiation was reported
    spills = {k: v for k, v in kernels.items() if v}
    assert not spills, spills

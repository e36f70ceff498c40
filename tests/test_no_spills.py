"""Register-spill guard (CPU only): every HIP source of the library is
compiled for gfx950 with the compiler's kernel resource report, and no
kernel may spill registers or use scratch memory. A spill turns register
traffic into per-lane memory traffic inside the hot loops; a change that
causes one should fail here, not show up later as a slowdown."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_quantized_gemm_amd import build_lib

HIPCC = build_lib.HIPCC
SOURCES = [s for s in build_lib.SOURCES + build_lib.PROBE_SOURCES if s.endswith(".hip")]


def _report(src: str, tmpdir: str) -> str:
    out = os.path.join(tmpdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *build_lib.COMMON, *build_lib.HIP_FLAGS, "-x", "hip", "-c",
           os.path.join(build_lib.CSRC, src), "-o", out, "--offload-device-only",
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{src}: compile failed\n{r.stderr[-2000:]}"
    return r.stderr


def _kernels(report: str):
    """(kernel, {field: value}) for every kernel in a resource report."""
    cur, name = {}, None
    for line in report.splitlines():
        m = re.search(r"remark:\s+(.*?)\s*\[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            if name:
                yield name, cur
            name, cur = text.split(":", 1)[1].strip(), {}
        elif ":" in text:
            k, v = text.rsplit(":", 1)
            cur[k.strip()] = v.strip()
    if name:
        yield name, cur


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)), reason="hipcc not found")
def test_no_kernel_spills_registers(tmp_path):
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        reports = dict(zip(SOURCES, ex.map(lambda s: _report(s, str(tmp_path)), SOURCES)))
    bad, seen = [], 0
    for src, rep in reports.items():
        for name, f in _kernels(rep):
            seen += 1
            vs = int(f.get("VGPRs Spill", "0"))
            ss = int(f.get("SGPRs Spill", "0"))
            scratch = int(f.get("ScratchSize [bytes/lane]", "0"))
            if vs or ss or scratch:
                bad.append(f"{src}: {name}: VGPR spill {vs}, SGPR spill {ss}, scratch {scratch} B/lane")
    assert seen > 50, f"only {seen} kernels in the reports: parsing failed?"
    assert not bad, "kernels spill registers:\n" + "\n".join(bad)

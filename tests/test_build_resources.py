"""Resource usage of every gfx950 kernel, from the compiler's kernel-resource-usage report (CPU only: hipcc
cross-compiles without a GPU). No kernel may spill registers or use private (scratch) memory, and the LDS of
every kernel must fit the 160 KiB of a CU. The report is printed, one kernel per line."""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD_PY = os.path.join(ROOT, "linear_attention_decay_amd", "build.py")

FIELDS = {
    "VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
    "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
    "LDS Size [bytes/block]": "lds",
}


def _demangle(name):
    try:
        return subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip() or name
    except OSError:
        return name


def resource_report(tmp_dir):
    spec = importlib.util.spec_from_file_location("_la_build", BUILD_PY)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = os.path.join(tmp_dir, "libresources.so")
    cmd = [hipcc, "-Rpass-analysis=kernel-resource-usage", *b.HIPCC_FLAGS, "-I", b.INCLUDE, *b.SRCS, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = _demangle(m.group(1))
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([^:]+?):\s*(-?\d+)\s", line + " ")
        if m and cur is not None and m.group(1).strip() in FIELDS:
            kernels[cur][FIELDS[m.group(1).strip()]] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) and not shutil.which("hipcc"),
                    reason="hipcc not available")
def test_no_kernel_spills_or_uses_scratch(tmp_path):
    kernels = resource_report(str(tmp_path))
    names = sorted(kernels)
    assert any("la_chunk_kernel<0>" in n for n in names), names
    assert any("la_short_kernel" in n for n in names), names
    for n in names:
        k = kernels[n]
        print(f"{n}: " + ", ".join(f"{f} {k.get(f)}" for f in FIELDS.values()), flush=True)
    for n in names:
        k = kernels[n]
        assert k.get("scratch") == 0, f"{n} uses {k.get('scratch')} bytes of scratch per lane"
        assert k.get("vgpr_spill") == 0, f"{n} spills {k.get('vgpr_spill')} VGPRs"
        assert k.get("sgpr_spill") == 0, f"{n} spills {k.get('sgpr_spill')} SGPRs"
        assert k.get("lds", 0) <= 160 * 1024, f"{n} needs {k.get('lds')} bytes of LDS"

"""Every gfx950 kernel of the library fits its registers without spilling."""
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_57_amd", "csrc")


@pytest.mark.parametrize("src", ["pa_attention.hip", "pa_cache.hip"])
def test_no_register_spills(src):
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-O3", "-std=c++17", "--cuda-device-only", "-c",
                        os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", r.stderr)]
    sspills = [int(x) for x in re.findall(r"SGPRs Spill: (\d+)", r.stderr)]
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(spills) == len(names)
    bad = [n for n, v, s in zip(names, spills, sspills) if v or s]
    assert not bad, f"kernels with spills: {bad}"
    assert not any(scratch), "kernels using scratch memory"

"""Properties of the compiled gfx950 kernels, checked on the CPU from hipcc output.

* No kernel spills registers or uses scratch memory (the float32 head_dim-128
  VALU worker may keep a few values in accumulation registers; the prefill tile
  worker may keep up to two scalar values in lanes of a vector register, which
  it writes once per workgroup and reads once per item).
* The attention workers and the merge contain no exec-mask regions: nothing
  inside them branches per lane (the one exception is the TILE worker's work
  ticket, taken by lane 0 between two barriers).  Their work loops call cross-lane operations
  (readfirstlane, readlane, shuffles, MFMA); a lane-dependent branch near such
  a loop let the compiler split the wavefront across loop iterations, which
  left lanes running with a stale work item.
"""
import importlib.util
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_57_amd", "csrc")


def device_flags():
    spec = importlib.util.spec_from_file_location("pa_build", os.path.join(ROOT, "paged_kv_cache_57_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.DEVICE_FLAGS


def compile_device(src, extra):
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", *device_flags(), "-O3", "-std=c++17",
                        "--cuda-device-only", os.path.join(CSRC, src), *extra],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return r


@pytest.mark.parametrize("src", ["pa_attention.hip", "pa_cache.hip"])
def test_no_register_spills(src):
    r = compile_device(src, ["-c", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"])
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", r.stderr)]
    sspills = [int(x) for x in re.findall(r"SGPRs Spill: (\d+)", r.stderr)]
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(spills) == len(names)
    # the float32 head_dim-128 VALU worker runs at one wavefront per SIMD and parks a few
    # values in accumulation registers (a spill with no scratch memory); no other kernel spills
    agpr_ok = [n for n, v, sc in zip(names, spills, scratch) if "valu_attn_kernelIfLi128E" in n and v <= 8 and sc == 0]
    lane_ok = [n for n, s, sc in zip(names, sspills, scratch) if "tile_attn_kernel" in n and s <= 2 and sc == 0]
    bad = [n for n, v, s in zip(names, spills, sspills) if (v and n not in agpr_ok) or (s and n not in lane_ok)]
    assert not bad, f"kernels with spills: {bad}"
    assert not any(scratch), "kernels using scratch memory"


def test_workers_have_no_per_lane_branches(tmp_path):
    asm = tmp_path / "attn.s"
    compile_device("pa_attention.hip", ["-S", "-o", str(asm)])
    text = asm.read_text()
    bodies = re.findall(r"^(_Z\S+):.*?^\.Lfunc_end", text, flags=re.S | re.M)
    funcs = re.split(r"^(?=_Z\S+:)", text, flags=re.M)
    checked = 0
    for f in funcs:
        m = re.match(r"(_Z\S+):", f)
        if not m or not re.search(r"(valu_attn|mfma_attn|tile_attn|merge)_kernel", m.group(1)):
            continue
        body = f.split(".Lfunc_end")[0]
        n = len(re.findall(r"\bs_and_saveexec_b64|\bs_andn2_saveexec_b64|\bs_or_saveexec_b64", body))
        if "tile_attn" in m.group(1) or "valu_attn" in m.group(1):
            # the single exception: thread 0 takes the workgroup's next work ticket, between two
            # barriers; the region holds the atomic and the store of its result to LDS, and the
            # mask is restored right after it
            assert n <= 1, f"{m.group(1)} has {n} exec-mask regions"
            if n:
                ops, restored = _ticket_region(body)
                assert restored, f"{m.group(1)}: the ticket region's join block does not restore the mask first"
                assert "global_atomic_add" in ops and "ds_write_b32" in ops, f"{m.group(1)}: {ops}"
                assert all(o.startswith(("s_", "v_mov", "global_atomic_add", "ds_write_b32")) for o in ops), ops
        else:
            assert n == 0, f"{m.group(1)} has {n} exec-mask regions"
        checked += 1
    assert checked >= 8 and bodies is not None

def _ticket_region(body):
    """The instructions of the one exec-mask region of a worker (wherever the compiler placed its
    block), and whether the block it joins starts by restoring the saved mask."""
    lines = [ln.split(";")[0].strip() for ln in body.splitlines()]  # without comments
    lines = [ln for ln in lines if ln]
    i = next(k for k, ln in enumerate(lines) if ln.startswith("s_and_saveexec_b64"))
    saved = re.match(r"s_and_saveexec_b64\s+(s\[\d+:\d+\])", lines[i]).group(1)
    skip = re.match(r"s_cbranch_execz\s+(\.LBB\S+)", lines[i + 1])
    assert skip, lines[i + 1]
    ops, k, join = [], i + 2, None
    while k < len(lines):
        ln = lines[k]
        if ln.endswith(":") and ln.startswith(".LBB"):  # falls through into the next block
            join = ln[:-1]
            break
        op = ln.split()[0]
        if op == "s_branch":
            join = ln.split()[1]
            break
        if not op.startswith("."):
            ops.append(op)
        k += 1
    if join != skip.group(1):
        return ops, False
    j = lines.index(join + ":")
    first = next(ln for ln in lines[j + 1:] if not ln.startswith("."))
    return ops, first.replace(" ", "") == f"s_or_b64exec,exec,{saved}"

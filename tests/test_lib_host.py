"""CPU tests of libpa: exports, host-side argument checks, allocator parity with the mirror.

Nothing here launches a kernel: every call either is pure host code (the
allocator) or fails its argument checks before any device work.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from oracle import allocator as mirror
from tests._lib import ensure_built
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_cache_57_amd as pa
    return pa


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_probe_library_exports_its_header(pa):
    # the measurement-only probes (page reads, LDS reads) live in libpa_probe.so, not in the product library
    from paged_kv_cache_57_amd import build as _b
    hdr = open(os.path.join(ROOT, "include", "pa_probe.h")).read()
    names = set(re.findall(r"\b(pa_probe_\w+)\(", hdr))
    assert names == {"pa_probe_read_pages", "pa_probe_lds_read", "pa_probe_last_error"}
    nm = subprocess.run(["nm", "-D", "--defined-only", _b.PROBE_LIB], capture_output=True, text=True).stdout
    assert names <= set(re.findall(r"\bT (pa_probe_\w+)", nm))
    main = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True).stdout
    assert "read_pages" not in main and "lds_read" not in main


def test_library_exports_every_declared_function(pa):
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(pa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pa_\w+)", nm))
    assert set(names) <= exported
    assert set(pa.EXPORTS) == set(names)          # the binding declares exactly the header's functions
    # every entry point outside the allocator and the composer (wrapped by pa.Allocator and
    # pa.SplitFuse) is a package function
    for n in names:
        if not n.startswith(("pa_alloc_", "pa_seq_", "pa_sf_")):
            assert callable(getattr(pa, n, None)), n


def test_abi_version(pa):
    assert pa.pa_abi_version() == 1


def test_host_argument_checks_fail_before_any_launch(pa):
    lib = pa._binding._lib
    # head_dim 96, block_size 8, GQA mismatch, bad dtype: rejected on the host
    st = lib.pa_forward(None, None, None, None, None, 1, None, None, 1, 1, 1, 1, 4, 4, 96, 16, 8, 1.0, 1,
                        None, 0, None, None)
    assert st == pa.PA_ERR_UNSUPPORTED and "head_dim" in pa.pa_last_error()
    st = lib.pa_forward(None, None, None, None, None, 1, None, None, 1, 1, 1, 1, 4, 4, 128, 8, 8, 1.0, 1,
                        None, 0, None, None)
    assert st == pa.PA_ERR_UNSUPPORTED and "block_size" in pa.pa_last_error()
    st = lib.pa_forward(None, None, None, None, None, 8, None, None, 1, 1, 1, 1, 4, 4, 128, 16, 8, 1.0, 0,
                        None, 0, None, None)
    assert st == pa.PA_ERR_INVALID and "NULL" in pa.pa_last_error()   # float32 at head_dim 128 is supported
    st = lib.pa_forward(None, None, None, None, None, 1, None, None, 1, 1, 1, 1, 6, 4, 128, 16, 8, 1.0, 1,
                        None, 0, None, None)
    assert st == pa.PA_ERR_INVALID
    st = lib.pa_forward(None, None, None, None, None, 1, None, None, 1, 1, 1, 1, 4, 4, 128, 16, 8, 1.0, 1,
                        None, 0, None, None)
    assert st == pa.PA_ERR_INVALID and "NULL" in pa.pa_last_error()
    st = lib.pa_forward(None, None, None, None, None, 1, None, None, 1, 1, 2, 1, 4, 4, 128, 16, 8, 1.0, 1,
                        None, 0, None, None)
    assert st == pa.PA_ERR_INVALID and "max_q_len" in pa.pa_last_error()
    st = lib.pa_reshape_and_cache(None, None, None, None, None, 4, 8, 2, 128, 16, 7, None, None)
    assert st == pa.PA_ERR_UNSUPPORTED
    st = lib.pa_copy_blocks(None, None, None, -1, 8, 2, 128, 16, 1, None, None)
    assert st == pa.PA_ERR_INVALID
    # empty work is a no-op success
    assert lib.pa_copy_blocks(None, None, None, 0, 8, 2, 128, 16, 1, None, None) == pa.PA_OK
    assert lib.pa_reshape_and_cache(None, None, None, None, None, 0, 8, 2, 128, 16, 1, None, None) == pa.PA_OK


def test_workspace_bytes_grow_with_split_contexts(pa):
    small = pa.pa_forward_workspace_bytes(2, 2, 1, 4, 4, 64, 100, pa.PA_F32)
    big = pa.pa_forward_workspace_bytes(2, 2, 1, 4, 4, 64, 5000, pa.PA_F32)
    assert small > 0 and big > small
    assert pa.pa_forward_workspace_bytes(2, 2, 1, 6, 4, 64, 100, pa.PA_F32) == 0


# ---------------------------------------------------------------- allocator parity

def random_ops(seed, n_ops=4000, n_blocks=48, block_size=4):
    rng = np.random.default_rng(seed)
    ops = []
    for _ in range(n_ops):
        k = rng.integers(0, 100)
        sid = int(rng.integers(0, 24))
        if k < 18:
            ops.append(("create", sid, int(rng.integers(0, 3 * block_size * 3))))
        elif k < 30:
            ops.append(("fork", sid, int(rng.integers(0, 24))))
        elif k < 75:
            ops.append(("append", sid))
        elif k < 88:
            ops.append(("free", sid))
        elif k < 94:
            ops.append(("can", int(rng.integers(0, n_blocks * block_size + 20))))
        else:
            ops.append(("table", sid))
    return ops


def run_mirror(ops, n_blocks, block_size, watermark, order):
    a = mirror.Allocator(n_blocks, block_size, watermark, order)
    out = []
    for op in ops:
        try:
            if op[0] == "create":
                a.create(op[1], op[2]); out.append((0,))
            elif op[0] == "fork":
                a.fork(op[1], op[2]); out.append((0,))
            elif op[0] == "append":
                slot, cow = a.append_slot(op[1])
                out.append((0, slot) + (cow if cow else (-1, -1)))
            elif op[0] == "free":
                a.free_seq(op[1]); out.append((0,))
            elif op[0] == "can":
                out.append((0, a.can_allocate(op[1])))
            elif op[0] == "table":
                out.append((0,) + tuple(a.block_table(op[1])))
        except mirror.NoBlocks:
            out.append((-3,))
        except KeyError:
            out.append((-5,))
        except ValueError:
            out.append((-1,))
        out[-1] = out[-1] + (a.num_free(),)
    return out


def run_ctypes(pa, ops, n_blocks, block_size, watermark, order):
    a = pa.Allocator(n_blocks, block_size, watermark, order)
    out = []
    for op in ops:
        try:
            if op[0] == "create":
                a.create(op[1], op[2]); out.append((0,))
            elif op[0] == "fork":
                a.fork(op[1], op[2]); out.append((0,))
            elif op[0] == "append":
                slot, cow = a.append_slot(op[1])
                out.append((0, slot) + (cow if cow else (-1, -1)))
            elif op[0] == "free":
                a.free(op[1]); out.append((0,))
            elif op[0] == "can":
                out.append((0, a.can_allocate(op[1])))
            elif op[0] == "table":
                out.append((0,) + tuple(a.block_table(op[1])))
        except pa.PAError as e:
            out.append((e.status,))
        out[-1] = out[-1] + (a.num_free(),)
    a.close()
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_allocator_matches_mirror_bit_for_bit(pa, seed):
    n_blocks, bs = 48, 4
    order = np.random.default_rng(100 + seed).permutation(n_blocks)
    ops = random_ops(seed, n_blocks=n_blocks, block_size=bs)
    want = run_mirror(ops, n_blocks, bs, 0.1, order)
    got = run_ctypes(pa, ops, n_blocks, bs, 0.1, order)
    assert got == want
    statuses = {r[0] for r in want}
    assert {0, -3, -5, -1} <= statuses          # every outcome kind was exercised


def test_allocator_batch_calls_match_single_calls(pa):
    a, b = pa.Allocator(64, 16), pa.Allocator(64, 16)
    for x in (a, b):
        x.create(0, 40)
        for c in (1, 2, 3):
            x.fork(0, c)
    slots, pairs = a.append_slots([0, 1, 2, 3])
    single = [b.append_slot(s) for s in (0, 1, 2, 3)]
    assert list(slots) == [s for s, _ in single]
    assert [tuple(p) for p in pairs] == [c for _, c in single if c]
    tab = a.block_tables([0, 1, 2, 3], 5)
    assert tab.shape == (4, 5) and (tab[:, 3:] == -1).all()
    assert [list(r[:3]) for r in tab] == [b.block_table(s) for s in (0, 1, 2, 3)]
    assert list(a.slots(2, 38, 3)) == list(b.slots(2, 38, 3))
    assert a.num_tokens(3) == 41
    with pytest.raises(pa.PAError):
        a.slots(2, 40, 2)


def test_allocator_create_rejects_bad_free_order(pa):
    with pytest.raises(pa.PAError):
        pa.Allocator(4, 16, 0.0, [0, 1, 1, 3])
    with pytest.raises(pa.PAError):
        pa.Allocator(4, 16, 1.5)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_allocator_under_address_and_ub_sanitizers():
    out_dir = os.path.join(ROOT, "tests", "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "alloc_driver_asan")
    csrc = os.path.join(ROOT, "paged_kv_cache_57_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "alloc_driver.cpp"), os.path.join(csrc, "pa_alloc.cpp"),
                    os.path.join(csrc, "pa_status.cpp"), "-o", exe], check=True)
    n_blocks, bs = 40, 4
    order = np.random.default_rng(7).permutation(n_blocks)
    ops = random_ops(11, n_ops=3000, n_blocks=n_blocks, block_size=bs)
    script = [f"order {n_blocks} {bs} 0.05 " + " ".join(map(str, order))]
    for op in ops:
        script.append(" ".join(map(str, op)))
        script.append("nfree")
    r = subprocess.run([exe], input="\n".join(script) + "\n", capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert lines[0] == "0"
    got = []
    for i in range(len(ops)):
        res = tuple(int(x) for x in lines[1 + 2 * i].split())
        nfree = int(lines[2 + 2 * i])
        if ops[i][0] == "table" and res[0] == 0:
            res = (0,) + res[2:]
        elif ops[i][0] in ("table",):
            res = res[:1]
        elif ops[i][0] == "append" and res[0] != 0:
            res = res[:1]
        got.append(res + (nfree,))
    assert got == run_mirror(ops, n_blocks, bs, 0.05, order)


def test_shared_prefix_and_rope_argument_checks(pa):
    """pa_forward_shared and pa_rope_reshape_and_cache reject bad arguments on the host
    (the fake device addresses below are never touched: every call fails a check first)."""
    lib = pa._binding._lib
    fake = ctypes.c_void_p(1 << 20)

    def shared(groups, ng, hq, hkv, d, dtype, ws_bytes=1 << 30, S=4, T=4):
        return lib.pa_forward_shared(fake, fake, fake, fake, fake, 8, fake, fake, groups, ng, S, T, 1, 100, hq, hkv,
                                     d, 16, 64, 1.0, dtype, fake, ws_bytes, None, None)
    assert shared(fake, 1, 4, 4, 64, pa.PA_F32) == pa.PA_ERR_UNSUPPORTED and "bfloat16" in pa.pa_last_error()
    assert shared(fake, 1, 32, 2, 128, pa.PA_BF16) == pa.PA_ERR_UNSUPPORTED      # 16 query heads per KV head
    assert shared(fake, -1, 4, 4, 128, pa.PA_BF16) == pa.PA_ERR_INVALID and "group" in pa.pa_last_error()
    assert shared(None, 2, 4, 4, 128, pa.PA_BF16) == pa.PA_ERR_INVALID
    assert shared(fake, 5, 4, 4, 128, pa.PA_BF16) == pa.PA_ERR_INVALID          # more groups than sequences
    assert shared(fake, 1, 4, 4, 128, pa.PA_BF16, ws_bytes=256) == pa.PA_ERR_INVALID and "workspace" in pa.pa_last_error()
    plain = pa.pa_forward_workspace_bytes(4, 4, 1, 4, 4, 128, 100, pa.PA_BF16)
    with_groups = pa.pa_forward_shared_workspace_bytes(4, 2, 4, 1, 4, 4, 128, 100, pa.PA_BF16)
    assert with_groups > plain and pa.pa_forward_shared_workspace_bytes(-1, 0, 4, 1, 4, 4, 128, 100, 1) == 0

    def rope(maxpos, d, cos=fake, T=3):
        return lib.pa_rope_reshape_and_cache(fake, fake, fake, fake, fake, fake, fake, fake, cos, fake, maxpos, T, 4, 2,
                                             8, d, 16, pa.PA_BF16, None, None)
    assert rope(0, 128) == pa.PA_ERR_INVALID
    assert rope(10, 96) == pa.PA_ERR_UNSUPPORTED
    assert rope(10, 128, cos=None) == pa.PA_ERR_INVALID and "NULL" in pa.pa_last_error()
    assert rope(10, 128, T=0) == pa.PA_OK                                       # nothing to do, nothing launched

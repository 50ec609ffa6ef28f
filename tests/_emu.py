"""Builds and drives the CPU kernel emulator (tests/emu) — CPU tests only.

The emulator compiles the library's own kernel sources for the host with a
stand-in HIP header and AddressSanitizer/UBSan, then runs the C-ABI entry
points on exact-size heap buffers.  Any out-of-bounds access in a kernel
aborts with the source line, on the CPU.
"""
import os
import subprocess
import tempfile

import numpy as np

from tests.conftest import ROOT

EXE = os.path.join(ROOT, "tests", "_build", "emu_main")
CLANG = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "paged_kv_cache_57_amd", "csrc")
SOURCES_HIP = ["pa_attention.hip", "pa_cache.hip"]


def available():
    return os.path.exists(CLANG)


def build(force=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES_HIP] + [os.path.join(CSRC, "pa_status.cpp")]
    emu = [os.path.join(ROOT, "tests", "emu", f) for f in ("emu_runtime.cpp", "emu_main.cpp", "hip/hip_runtime.h")]
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + [os.path.join(ROOT, "include", "pa.h")]
    if not force and os.path.exists(EXE):
        t = os.path.getmtime(EXE)
        if all(os.path.getmtime(f) < t for f in srcs + emu + hdrs):
            return EXE
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = f"{EXE}.{os.getpid()}.tmp"
    # -fno-honor-nans as in the device build: the compiler may then assume no float is NaN,
    # and the kernels' NaN-sensitive tests must survive that assumption here too
    cmd = [CLANG, "-std=c++20", "-O1", "-g", "-fno-honor-nans", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "tests", "emu"), "-I", os.path.join(ROOT, "include"),
           "-x", "c++", *[os.path.join(CSRC, s) for s in SOURCES_HIP], "-x", "none",
           os.path.join(CSRC, "pa_status.cpp"), emu[0], emu[1], "-lpthread", "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, EXE)  # atomic: concurrent test workers each build their own file
    return EXE


def _run(mode, blob, out_bytes, timeout=600):
    with tempfile.TemporaryDirectory() as d:
        fi, fo = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fi, "wb") as f:
            for b in blob:
                f.write(np.ascontiguousarray(b).tobytes())
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
        r = subprocess.run([EXE, mode, fi, fo], capture_output=True, text=True, timeout=timeout, env=env)
        if r.returncode != 0:
            raise RuntimeError(f"emulator {mode} failed ({r.returncode}):\n{r.stderr[-6000:]}")
        data = open(fo, "rb").read()
    assert len(data) == out_bytes + 4, (len(data), out_bytes)
    return data[:out_bytes], int(np.frombuffer(data[out_bytes:], np.int32)[0])


def dtype_code(dt):
    return 0 if dt == "f32" else 1


def forward(w, q, kp, vp):
    """Emulated pa_forward on host arrays (float32 or bf16 bit patterns); returns (out, status)."""
    es = 4 if w.dtype == "f32" else 2
    hdr = np.array([dtype_code(w.dtype), w.num_seqs, w.num_tokens, w.max_q_len, w.max_context_len,
                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_blocks, w.max_blocks_per_seq], np.int32)
    blob = [hdr, np.array([w.scale], np.float32), q, kp, vp, w.block_tables.astype(np.int32),
            w.context_lens.astype(np.int32), w.query_start_loc.astype(np.int32)]
    n = w.num_tokens * w.num_q_heads * w.head_dim
    raw, st = _run("forward", blob, n * es)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    return np.frombuffer(raw, dt).reshape(w.num_tokens, w.num_q_heads, w.head_dim), st


def forward_shared(w, q, kp, vp, groups):
    """Emulated pa_forward_shared; groups: int [G, 3] (first sequence, members, shared keys)."""
    es = 4 if w.dtype == "f32" else 2
    groups = np.ascontiguousarray(np.asarray(groups, np.int32).reshape(-1, 3))
    hdr = np.array([dtype_code(w.dtype), w.num_seqs, w.num_tokens, w.max_q_len, w.max_context_len,
                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_blocks, w.max_blocks_per_seq], np.int32)
    blob = [hdr, np.array([w.scale], np.float32), q, kp, vp, w.block_tables.astype(np.int32),
            w.context_lens.astype(np.int32), w.query_start_loc.astype(np.int32),
            np.array([groups.shape[0]], np.int32), groups]
    n = w.num_tokens * w.num_q_heads * w.head_dim
    raw, st = _run("forward_shared", blob, n * es)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    return np.frombuffer(raw, dt).reshape(w.num_tokens, w.num_q_heads, w.head_dim), st


def reshape_and_cache(dtype, key, val, kp, vp, slots):
    T, hkv, d = key.shape
    nb = kp.shape[0]
    hdr = np.array([dtype_code(dtype), T, nb, hkv, d], np.int32)
    raw, st = _run("reshape", [hdr, key, val, kp, vp, np.asarray(slots, np.int64)], kp.nbytes + vp.nbytes)
    return (np.frombuffer(raw[:kp.nbytes], kp.dtype).reshape(kp.shape),
            np.frombuffer(raw[kp.nbytes:], vp.dtype).reshape(vp.shape), st)


def copy_blocks(dtype, kp, vp, pairs):
    pairs = np.asarray(pairs, np.int32).reshape(-1, 2)
    nb, hkv = kp.shape[0], kp.shape[1]
    d = vp.shape[2]
    hdr = np.array([dtype_code(dtype), pairs.shape[0], nb, hkv, d], np.int32)
    raw, st = _run("copy", [hdr, kp, vp, pairs], kp.nbytes + vp.nbytes)
    return (np.frombuffer(raw[:kp.nbytes], kp.dtype).reshape(kp.shape),
            np.frombuffer(raw[kp.nbytes:], vp.dtype).reshape(vp.shape), st)


def rope_reshape_and_cache(dtype, q, key, val, kp, vp, slots, positions, cos, sin):
    """Emulated pa_rope_reshape_and_cache (q rotated in place); returns (q_out, k_pool, v_pool, status)."""
    T, hq, d = q.shape
    hkv, nb = key.shape[1], kp.shape[0]
    hdr = np.array([dtype_code(dtype), T, hq, hkv, d, nb, cos.shape[0]], np.int32)
    blob = [hdr, q, key, val, kp, vp, np.asarray(slots, np.int64), np.asarray(positions, np.int32),
            np.ascontiguousarray(cos, np.float32), np.ascontiguousarray(sin, np.float32)]
    raw, st = _run("rope", blob, q.nbytes + kp.nbytes + vp.nbytes)
    qo = np.frombuffer(raw[:q.nbytes], q.dtype).reshape(q.shape)
    k = np.frombuffer(raw[q.nbytes:q.nbytes + kp.nbytes], kp.dtype).reshape(kp.shape)
    v = np.frombuffer(raw[q.nbytes + kp.nbytes:], vp.dtype).reshape(vp.shape)
    return qo, k, v, st


def forward_sparse(w, q, pages_k, pages_v, used):
    """Emulated pa_forward on a full-size zeroed pool holding only the ``used`` blocks' pages."""
    es = 4 if w.dtype == "f32" else 2
    hdr = np.array([dtype_code(w.dtype), w.num_seqs, w.num_tokens, w.max_q_len, w.max_context_len,
                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_blocks, w.max_blocks_per_seq], np.int32)
    blob = [hdr, np.array([w.scale], np.float32), q, np.array([len(used)], np.int32),
            np.asarray(used, np.int32), pages_k, pages_v, w.block_tables.astype(np.int32),
            w.context_lens.astype(np.int32), w.query_start_loc.astype(np.int32)]
    n = w.num_tokens * w.num_q_heads * w.head_dim
    raw, st = _run("forward_sparse", blob, n * es, timeout=3600)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    return np.frombuffer(raw, dt).reshape(w.num_tokens, w.num_q_heads, w.head_dim), st

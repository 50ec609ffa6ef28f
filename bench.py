#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

One step is one pass of the path over one batch of synthetic input, with all
inputs resident in device memory before timing starts:

* splitfuse (default): a Dynamic-SplitFuse forward — the cache write of all
  2048 new tokens through their slots, then one paged-attention pass over two
  causal 512-token prefill chunks (prior context uniform in [0, 8192]) and
  1024 single-token decodes (context uniform in [128, 4096]); 32 heads of dim
  128, bfloat16, 16-token pages.  value = query tokens per second.
* llama7b / gqa70b / gqa70b_long: decode-only passes (batch 64 MHA 32x128;
  batch 32 GQA 64/8 at 2048 keys; one GQA sequence of 32768 keys).  value =
  KV bytes read per second.
* sampling: the parallel-sampling workflow (16 prompts x 4 branches sharing
  prompt pages, copy-on-write, 64 decode rows per step); value = decode
  tokens per second over the timed steps, allocator and uploads included.
  --shared-prefix attends with pa_forward_shared (a prompt's pages are read
  once for its four branches).  A step is one pa_decode_step call (allocator,
  one upload, copies, cache write and attention); --composed-step issues the
  same operations one by one from Python.
* splitfuse_rope: the same pass with the rotary embedding fused into the cache
  write (pa_rope_reshape_and_cache rotates q and the new keys at their
  positions; the forward reads the rotated q).
* copy / read / lds: calibration lines, not the path — a 4 GiB device copy,
  every 4 KiB page of a pool (4 GiB, or --read-gib) read once in random order
  (the measurement library's pa_probe_read_pages), and 16-byte LDS reads on
  every compute unit (pa_probe_lds_read),
  the attainable HBM rates the kernels' fractions are set against.

The roofline object describes the dominant kernel, timed with HIP events
recorded on the stream it runs on (pa_set_stage_events), against MI355X's
8 TB/s HBM (decode workers) or 2.5 PFLOP/s dense bf16 MFMA at 2.4 GHz (the
prefill tile worker); for a decode worker it also carries the page-read
probe's rate over passes of the same size, measured in the same run, and the
kernel's fraction of it.  step_ms gives the median / min / max device time of
the timed steps, clock the shader clock sampled while they ran.
cpu_baseline times the fp64 CPU oracle on a bounded sample of the same pass
(query rows drawn uniformly from the pass's rows) on this host.

    python bench.py [--workload splitfuse] [--steps 100] [--warmup 5] [--gpus 1] [--rotate 1]

--rotate 1 keeps one pool for every step: a pass that fits the 256 MB
Infinity Cache (MALL) then finds its pages there ("kv_residency": "warm");
by default enough pool copies are cycled that none can ("cold").
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn KV-read GB/s (% HBM peak); SplitFuse mixed-batch tokens/s"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
MALL_BYTES = 256 << 20
STAGES = ("plan", "valu_worker", "mfma_worker", "tile_worker", "merge")
WORKERS = ("valu_worker", "mfma_worker", "tile_worker")


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def new(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        self.events += out
        return out

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def close(self):
        for e in self.events:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))
        self.events = []


# rocprofv3 kernel names of each worker, for looking up counter results
DOMINANT_KERNEL = {("valu_worker", "bf16", 128): "valu_attn_kernel<unsigned short, 128>",
                   ("valu_worker", "bf16", 64): "valu_attn_kernel<unsigned short, 64>",
                   ("valu_worker", "f32", 64): "valu_attn_kernel<float, 64>",
                   ("mfma_worker", "bf16", 128): "mfma_attn_kernel<128>",
                   ("mfma_worker", "bf16", 64): "mfma_attn_kernel<64>",
                   ("mfma_worker", "f32", 64): "mfma_attn_kernel<64>",
                   ("tile_worker", "bf16", 128): "tile_attn_kernel<128>",
                   ("tile_worker", "bf16", 64): "tile_attn_kernel<64>",
                   ("tile_worker", "f32", 64): "tile_attn_kernel<64>"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_57_amd", "csrc", "pa_attention.hip")


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a copy of known size),
    or None when there is none or the kernel source changed since it was taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    for e in rec.get("entries", []):
        if e["workload"] == workload and e["kernel"] == kernel:
            return round(e["fetch_kib"] * 1024 * rec["fetch_scale"] + e["write_kib"] * 1024 * rec["write_scale"])
    return None


def build_workload(name):
    import workloads as W
    return {"splitfuse": lambda: W.splitfuse_mixed(0),
            "splitfuse_rope": lambda: W.splitfuse_mixed(0),
            "llama7b": lambda: W.llama7b_decode(0),
            "gqa70b": lambda: W.gqa70b_decode(0),
            "gqa70b_long": lambda: W.gqa70b_long_decode(0),
            "tiny": lambda: W.tiny_decode(0)}[name]()


def kv_token_bytes(w):
    return 2 * w.num_kv_heads * w.head_dim * (4 if w.dtype == "f32" else 2)


def work_split(w):
    """Algorithmic work of one pass, split by the worker that does it.

    A sequence goes where the library's planner sends it: decode rows with one
    query head per KV head (and everything in float32) to the VALU worker;
    sequences with at most 16 rows per KV head (q_len x group size: GQA decode,
    short chunks) to the MFMA worker; longer prefill chunks to the tile worker.
    Bytes are the KV pages a worker's rows must read (each context key once
    per KV head: 2 * Hkv * d * elem bytes per key); FLOPs count QK^T and PV
    over the keys each row of a multi-row chunk may see (4 d Hq (pos + 1)).
    """
    ql = np.diff(w.query_start_loc).astype(np.int64)
    L = w.context_lens.astype(np.int64)
    G = w.num_q_heads // w.num_kv_heads
    live = (ql >= 1) & (L >= 1)
    valu = live & (((ql == 1) & (G == 1)) if w.dtype == "bf16" else True)
    mfma = live & ~valu & (ql * G <= 16)
    tile = live & ~valu & ~mfma
    work = {}
    for name, sel in (("valu_worker", valu), ("mfma_worker", mfma), ("tile_worker", tile)):
        flops = 0
        for q, Ls in zip(ql[sel & (ql > 1)], L[sel & (ql > 1)]):
            pos = Ls - q + np.arange(q)
            flops += 4 * w.head_dim * w.num_q_heads * int((pos + 1).sum())
        work[name] = {"bytes": int(L[sel].sum()) * kv_token_bytes(w), "flops": flops}
    return work


def host_info():
    """The host the CPU baseline ran on: CPU model, BLAS pools and library versions."""
    import platform

    import torch
    info = {"cpu_model": None, "host_cpus": len(os.sched_getaffinity(0)), "python": platform.python_version(),
            "numpy": np.__version__, "torch": torch.__version__, "blas": []}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import threadpoolctl
        info["blas"] = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                        for p in threadpoolctl.threadpool_info()]
    except Exception:
        pass
    return info


def cpu_baseline(w, q, kc, vc, budget_s):
    """The fp64 oracle on a bounded sample of the pass: query rows drawn uniformly
    from all of the pass's rows (so prefill-chunk rows and decode rows come in
    the pass's own proportion), each attended at its position over host copies
    of its sequence's pages.  Only the oracle calls are timed."""
    import torch

    from oracle import attention as oattn
    ql = np.diff(w.query_start_loc)
    seq_of_row = np.repeat(np.arange(w.num_seqs), ql)
    rng = np.random.default_rng(123)
    order = rng.permutation(w.num_tokens)

    def raw(t):
        t = t.detach().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    pages = {}
    spent = 0.0
    rows = chunk_rows = 0
    kv_bytes = 0
    for t in order:
        s = int(seq_of_row[t])
        Ls = int(w.context_lens[s])
        nb = (Ls + 15) // 16
        if s in pages:
            kp, vp = pages[s]
        else:
            ids = torch.from_numpy(w.block_tables[s, :nb].astype(np.int64)).to(kc.device)
            kp, vp = raw(kc.index_select(0, ids)), raw(vc.index_select(0, ids))
            if ql[s] > 1:
                pages[s] = (kp, vp)  # a prefill chunk's rows are drawn many times
        a, b = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        qh = raw(q[a:b])
        tab = np.arange(nb, dtype=np.int32)[None]
        t0 = time.perf_counter()
        oattn.paged_attention(qh, kp, vp, tab, np.array([Ls], np.int32), np.array([0, b - a], np.int32),
                              w.scale, w.dtype, tokens=[int(t) - a])
        spent += time.perf_counter() - t0
        rows += 1
        chunk_rows += int(ql[s] > 1)
        kv_bytes += (Ls - (b - 1 - int(t))) * kv_token_bytes(w)  # keys this row sees
        if spent >= budget_s:
            break
    host = host_info()
    threads = max([b["num_threads"] or 1 for b in host["blas"]] or [1])
    return {"rows": rows, "chunk_rows": chunk_rows, "seconds": spent, "kv_bytes": kv_bytes, "cores": threads,
            "host": host}


def copy_calibration(torch, dev, args, nbytes=4 << 30):
    """Device-to-device copy of a 4 GiB buffer: achievable HBM bandwidth, and the
    known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbps = 2 * nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "device copy GB/s (read + write)", "value": round(gbps, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": "copy_4GiB", "bytes_read": nbytes,
                                                      "bytes_written": nbytes},
                      "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}), flush=True)


class ProbeLib:
    """ctypes face of libpa_probe.so, the measurement-only page-read probe."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "paged_kv_cache_57_amd", "libpa_probe.so")
        if not os.path.exists(path):
            raise SystemExit(f"{path} is not built")
        self.lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        self.lib.pa_probe_read_pages.restype = i32
        self.lib.pa_probe_read_pages.argtypes = [vp, i64, vp, i32, vp, i32, i32, i32, vp, vp]
        self.lib.pa_probe_lds_read.restype = i32
        self.lib.pa_probe_lds_read.argtypes = [vp, i32, i32, i32, vp]
        self.lib.pa_probe_last_error.restype = ctypes.c_char_p

    def read_pages(self, torch, pool, page_ids, sink, grid, pages_in_flight, mode, status):
        st = self.lib.pa_probe_read_pages(pool.data_ptr(), pool.numel() * pool.element_size(), page_ids.data_ptr(),
                                          page_ids.numel(), sink.data_ptr(), grid, pages_in_flight, mode,
                                          status.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(self.lib.pa_probe_last_error().decode())


    def lds_read(self, torch, sink, grid, waves, iters):
        st = self.lib.pa_probe_lds_read(sink.data_ptr(), grid, waves, iters, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(self.lib.pa_probe_last_error().decode())


READ_MODES = {0: "plain", 1: "nontemporal", 2: "into_lds"}
READ_MODES.update({3 + a: f"buffer_cpol_{c}" for a, c in enumerate((0, 1, 2, 3, 16, 17, 18, 19))})


def lds_calibration(torch, dev, args):
    """LDS read rate: --lds-waves wavefronts per workgroup (4, 8, 16) on one workgroup
    per CU read 16-byte pieces of a 64 KiB LDS array; bytes read / kernel time."""
    probe = ProbeLib()
    props = torch.cuda.get_device_properties(dev)
    grid, waves, iters = props.multi_processor_count, args.lds_waves, 4096
    sink = torch.empty(grid * 64 * waves, dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        probe.lds_read(torch, sink, grid, waves, iters)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(args.steps):
        t0.record()
        probe.lds_read(torch, sink, grid, waves, iters)
        t1.record()
        t1.synchronize()
        times.append(t0.elapsed_time(t1))
    ms = float(np.median(times))
    nbytes = grid * waves * iters * 8 * 1024
    tbps = nbytes / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "LDS read TB/s (16-byte reads, whole GPU)", "value": round(tbps, 2), "unit": "TB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
                      "data": "synthetic", "config": {"workload": f"lds_read_{waves}waves", "workgroups": grid,
                                                      "waves_per_workgroup": waves, "bytes": nbytes},
                      "per_cu_GBps": round(tbps * 1e3 / grid, 1)}), flush=True)


def read_calibration(torch, pa, dev, args):
    """4 KiB pages of a 4 GiB pool read in a seeded random order with 16-byte loads,
    --read-pif pages per wavefront in flight (default 2, the decode workers' depth),
    --read-mode loads (0 plain, 1 non-temporal, 2 into LDS): the rate the decode
    workers' page reads could reach if they did no arithmetic.  By default a step
    reads every page once; with --read-mib M a step reads the next M MiB of the
    order (successive steps take disjoint slices, so none finds its pages in the
    256 MB Infinity Cache), the rate a pass of that size can reach.  With
    --read-chunk-pages N the order is a random permutation of runs of N consecutive
    pages (0: every page in address order), read by neighbouring wavefronts at the
    same time.  --read-grid sets the workgroups (0: one wavefront per
    pages-in-flight run of the slice, at most 2048 workgroups)."""
    probe = ProbeLib()
    nbytes = args.read_gib << 30
    pool = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(7)
    npages = nbytes // 4096
    run = args.read_chunk_pages
    if run < 0 or (run and npages % run):
        raise SystemExit(f"--read-chunk-pages must be 0 or divide {npages}")
    if run == 0:
        ids = np.arange(npages, dtype=np.int64)
    else:
        runs = np.random.default_rng(5).permutation(npages // run).astype(np.int64)
        ids = (runs[:, None] * run + np.arange(run)[None, :]).reshape(-1)
    order = torch.from_numpy(ids.astype(np.int32)).to(dev)
    per = npages if not args.read_mib else min(npages, args.read_mib * 256)
    nslices = npages // per
    slices = [order[i * per:(i + 1) * per] for i in range(nslices)]
    pif, mode = args.read_pif, args.read_mode
    g = args.read_grid or min(2048, max(1, (per + 4 * pif - 1) // (4 * pif)))
    sink = torch.empty(g * 256, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        probe.read_pages(torch, pool, slices[i % nslices], sink, g, pif, mode, status)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(args.steps):
        t0.record()
        probe.read_pages(torch, pool, slices[(args.warmup + i) % nslices], sink, g, pif, mode, status)
        t1.record()
        t1.synchronize()
        times.append(t0.elapsed_time(t1))
    if int(status.item()) != 0:
        raise RuntimeError(f"pa_probe_read_pages flagged status {int(status.item())}")
    ms = float(np.median(times))
    gbps = per * 4096 / (ms * 1e-3) / 1e9
    name = f"read_pages_{args.read_gib}GiB" if per == npages else f"read_pages_{per * 4096 >> 20}MiB_of_{args.read_gib}GiB"
    if run != 1:
        name += "_in_address_order" if run == 0 else f"_runs_of_{run}"
    print(json.dumps({"metric": "random 4 KiB page reads GB/s", "value": round(gbps, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "ms_min": round(min(times), 4), "ms_max": round(max(times), 4),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
                      "data": "synthetic", "config": {"workload": name, "pages": per, "grid": g,
                                                      "pages_in_flight_per_wave": pif, "loads": READ_MODES[mode]},
                      "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}), flush=True)


def sampling_workflow(torch, pa, W, dev, args):
    """Parallel sampling with shared prompt pages: 16 prompts (lengths uniform in
    [1000, 4000]) written once and forked into 4 branches each; every decode step
    appends one token per branch in the host allocator, copies the pages it
    reports (copy-on-write of a shared partial page), writes the 64 new K/V
    through their slots and runs attention for the 64 rows.  warmup + steps
    decode steps are timed by the wall clock (host allocator work and uploads
    included), then EVENT_STEPS more steps run with HIP events around the
    forward's stages for its device time.  A step is one pa_decode_step call;
    with --composed-step, the same operations issued one by one from Python."""
    EVENT_STEPS = 16
    spec = W.parallel_sampling_spec(0)
    P, B, NB, H, d = len(spec.prompt_lens), spec.branches, spec.num_blocks, spec.heads, spec.head_dim
    total = args.warmup + args.steps + EVENT_STEPS
    n = P * B
    ks, vs = W.cache_shapes(NB, H, d, "bf16")
    gen = torch.Generator(device=dev).manual_seed(0)
    kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=dev), gen)
    vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=dev), gen)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    alloc = pa.Allocator(NB, 16, 0.0, spec.initial_free_order)
    ids = [p * B + b for p in range(P) for b in range(B)]
    for p, L in enumerate(spec.prompt_lens):
        alloc.create(p * B, int(L))
    slots = np.concatenate([alloc.slots(p * B, 0, int(L)) for p, L in enumerate(spec.prompt_lens)])
    knew = W.fill_normal(torch.empty((len(slots), H, d), dtype=torch.bfloat16, device=dev), gen)
    vnew = W.fill_normal(torch.empty((len(slots), H, d), dtype=torch.bfloat16, device=dev), gen)
    pa.pa_reshape_and_cache(knew, vnew, kc, vc, torch.from_numpy(slots.astype(np.int64)).to(dev), status)
    for p in range(P):
        for b in range(1, B):
            alloc.fork(p * B, p * B + b)
    del knew, vnew
    qs = W.fill_normal(torch.empty((total, n, H, d), dtype=torch.bfloat16, device=dev), gen)
    kst = W.fill_normal(torch.empty((total, n, H, d), dtype=torch.bfloat16, device=dev), gen)
    vst = W.fill_normal(torch.empty((total, n, H, d), dtype=torch.bfloat16, device=dev), gen)
    lens = np.repeat(spec.prompt_lens.astype(np.int32), B)
    max_ctx = int(lens.max()) + total
    cap_max = (max_ctx + 15) // 16
    qsl = torch.arange(n + 1, dtype=torch.int32, device=dev)
    cascade = args.shared_prefix
    groups = None
    if cascade:
        # each prompt's branches (consecutive sequences) share its full pages
        groups = torch.tensor([[p * B, B, 16 * (int(L) // 16)] for p, L in enumerate(spec.prompt_lens)],
                              dtype=torch.int32, device=dev)
        nbytes = pa.pa_forward_shared_workspace_bytes(n, P, n, 1, H, H, d, 16 * cap_max, pa.PA_BF16)
    else:
        nbytes = pa.pa_forward_workspace_bytes(n, n, 1, H, H, d, 16 * cap_max, pa.PA_BF16)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    # Every step stages its slots, context lengths, tables and copy pairs in a
    # pinned region of its own (no copy waits for the device) and uploads them
    # into one device buffer (stream order keeps a step's copy behind the last
    # step's kernels): the staging layout of pa_decode_step.
    stride = pa.pa_decode_step_staging_bytes(n, cap_max)
    up = torch.empty((total, stride), dtype=torch.uint8).pin_memory()
    dbuf = torch.empty(stride, dtype=torch.uint8, device=dev)
    o_lens, o_qsl = 8 * n, 12 * n
    o_pairs = (16 * n + 4 + 7) // 8 * 8
    o_tab = o_pairs + 8 * n
    d_slots = dbuf[:o_lens].view(torch.int64)
    d_lens = dbuf[o_lens:o_qsl].view(torch.int32)
    d_pairs = dbuf[o_pairs:o_tab].view(torch.int32).view(n, 2)
    d_tab = dbuf[o_tab:].view(torch.int32)
    cur = torch.cuda.current_stream(dev)
    ev = HipEvents()
    stage_ev = [ev.new(2 * len(STAGES)) for _ in range(EVENT_STEPS)]
    logical = []
    scale = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()

    def composed_step(i):
        h = up[i].numpy()
        ncow, L, cols, used = pa.pa_decode_step_stage(alloc, ids, cap_max, h)
        dbuf[:used].copy_(up[i, :used], non_blocking=True)
        if ncow:
            pa.pa_copy_blocks(kc, vc, d_pairs[:ncow], status, cur)
        pa.pa_reshape_and_cache(kst[i], vst[i], kc, vc, d_slots, status, cur)
        tables = d_tab[:n * cols].view(n, cols)
        if cascade:
            pa.pa_forward_shared(out, qs[i], kc, vc, tables, d_lens, qsl, groups, 1, L, scale, ws, status, cur)
        else:
            pa.pa_forward(out, qs[i], kc, vc, tables, d_lens, qsl, 1, L, scale, ws, status, cur)

    def native_step(i):
        pa.pa_decode_step(alloc, ids, out, qs[i], kst[i], vst[i], kc, vc, scale, cap_max, up[i], dbuf, ws,
                          groups=groups, dev_status=status, stream=cur)

    step = composed_step if args.composed_step else native_step
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the forward's device time, from events around its stages on extra steps
    first_ev = args.warmup + args.steps
    for j in range(EVENT_STEPS):
        pa.pa_set_stage_events(stage_ev[j])
        step(first_ev + j)
        logical.append(int(sum(alloc.num_tokens(s) for s in ids)))
    torch.cuda.synchronize()
    pa.pa_set_stage_events(None)
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item()):#x}")
    # the forward's kernels: the sum of its stage durations (the gaps the events add between them excluded)
    fwd_ms = [sum(ev.ms(e[2 * k], e[2 * k + 1]) for k in range(len(STAGES))) for e in stage_ev]
    ev.close()
    tok_bytes = 2 * H * d * 2
    logical_bytes = sum(logical) * tok_bytes
    # unique pages: every prompt token once, plus each branch's own decode tokens
    unique_bytes = sum((int(spec.prompt_lens.sum()) + n * (i + 1)) * tok_bytes for i in range(first_ev, total))
    fwd_s = sum(fwd_ms) * 1e-3
    ms_per_step = 1e3 * elapsed / args.steps
    fwd_ms_mean = 1e3 * fwd_s / EVENT_STEPS
    achieved = unique_bytes / fwd_s / 1e9
    print(json.dumps({
        "metric": "parallel sampling decode tokens/s (shared prompt pages, copy-on-write)",
        "value": round(n * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "parallel_sampling_16x4", "prompts": P, "branches": B, "q_heads": H, "kv_heads": H,
                   "head_dim": d, "block_size": 16, "pool_blocks": NB, "decode_steps": total,
                   "step": "composed from the single entry points" if args.composed_step else "pa_decode_step",
                   "forward": "pa_forward_shared (prompt pages read once per prompt)" if cascade else "pa_forward"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "pa_forward",
                     "kernel_ms": round(fwd_ms_mean, 4), "algorithmic_bytes": "unique KV pages per step"},
        "forward_logical_kv_GBps": round(logical_bytes / fwd_s / 1e9, 1),
        "forward_unique_kv_GBps": round(achieved, 1),
        "forward_share_of_step": round(fwd_ms_mean / ms_per_step, 4)}), flush=True)


class ClockSampler:
    """Samples the shader clock (the level sysfs pp_dpm_sclk marks current) every
    few milliseconds on a thread while the timed steps run."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self.levels = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            with open(self.path) as f:
                lines = f.read().splitlines()
        except OSError:
            return None, []
        cur, levels = None, []
        for line in lines:
            try:
                mhz = int(line.split(":", 1)[1].strip().split("Mhz")[0])
            except (IndexError, ValueError):
                continue
            levels.append(mhz)
            if line.rstrip().endswith("*"):
                cur = mhz
        return cur, levels

    def _run(self):
        while not self._stop.is_set():
            cur, levels = self._read()
            if cur is not None:
                self.samples.append(cur)
                self.levels = levels
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"source": "sysfs pp_dpm_sclk", "samples": 0}
        x = np.array(self.samples)
        return {"source": "sysfs pp_dpm_sclk (current level, sampled every 2 ms over the timed steps; "
                          "a run of a few ms also catches the ramp from idle)",
                "samples": int(x.size), "median_mhz": int(np.median(x)), "min_mhz": int(x.min()),
                "max_mhz": int(x.max()), "top_level_mhz": int(max(self.levels)) if self.levels else None,
                "peak_assumes_mhz": 2400}


def probe_ceiling(torch, dev, pass_bytes, steps=12, warmup=2, pif=4, mode=1, pool_bytes=4 << 30):
    """The page-read probe (non-temporal 16-byte loads, pif pages per wavefront in
    flight) over passes of the dominant kernel's size: random 4 KiB pages of a
    4 GiB pool, a different slice each step, timed with a HIP event between
    consecutive launches (launches back to back).  Returns (GB/s median, bytes per pass)."""
    probe = ProbeLib()
    pool = torch.empty(pool_bytes // 4, dtype=torch.int32, device=dev).fill_(7)
    npages = pool_bytes // 4096
    per = int(min(npages, max(1, pass_bytes // 4096)))
    order = torch.from_numpy(np.random.default_rng(5).permutation(npages).astype(np.int32)).to(dev)
    nslices = max(1, npages // per)
    g = min(2048, max(1, (per + 4 * pif - 1) // (4 * pif)))
    sink = torch.empty(g * 256, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(warmup):
        probe.read_pages(torch, pool, order[(i % nslices) * per:(i % nslices + 1) * per], sink, g, pif, mode, status)
    # launches back to back, an event between each two (the device time of each)
    ev[0].record()
    for i in range(steps):
        k = (warmup + i) % nslices
        probe.read_pages(torch, pool, order[k * per:(k + 1) * per], sink, g, pif, mode, status)
        ev[i + 1].record()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"pa_probe_read_pages flagged status {int(status.item())}")
    ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    del pool
    torch.cuda.empty_cache()
    return per * 4096 / (ms * 1e-3) / 1e9, per * 4096


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="splitfuse",
                    choices=["splitfuse", "splitfuse_rope", "llama7b", "gqa70b", "gqa70b_long", "tiny", "copy", "read", "lds",
                             "sampling"])
    ap.add_argument("--rotate", type=int, default=0, help="pool copies cycled per step (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-mib", type=int, default=0, help="read workload: MiB per step (0: the whole 4 GiB pool)")
    ap.add_argument("--read-pif", type=int, default=2, help="read workload: pages per wavefront in flight (1, 2, 4, 8)")
    ap.add_argument("--read-mode", type=int, default=0,
                    help="read workload: 0 plain, 1 non-temporal, 2 into-LDS loads, 3..10 buffer loads with the "
                         "cache-policy bits 0, 1, 2, 3, 16, 17, 18, 19")
    ap.add_argument("--read-gib", type=int, default=4, help="read workload: pool size in GiB")
    ap.add_argument("--lds-waves", type=int, default=8, help="lds workload: wavefronts per workgroup (4, 8, 16)")
    ap.add_argument("--read-grid", type=int, default=0, help="read workload: workgroups (0: by the slice size)")
    ap.add_argument("--read-chunk-pages", type=int, default=1,
                    help="read workload: pages per run of consecutive pages in the random order (0: address order)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="sampling workload: attend with pa_forward_shared, the branches of a prompt as one group")
    ap.add_argument("--composed-step", action="store_true",
                    help="sampling workload: issue a step's operations one by one instead of one pa_decode_step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_57_amd as pa
    import workloads as W

    dev = torch.device("cuda:0")
    if args.workload == "copy":
        return copy_calibration(torch, dev, args)
    if args.workload == "read":
        return read_calibration(torch, pa, dev, args)
    if args.workload == "lds":
        return lds_calibration(torch, dev, args)
    if args.workload == "sampling":
        if args.warmup + args.steps > 256:
            print("the sampling workflow runs at most 256 decode steps (warmup + steps)", file=sys.stderr)
            sys.exit(2)
        return sampling_workflow(torch, pa, W, dev, args)
    w = build_workload(args.workload)
    code = pa.PA_BF16 if w.dtype == "bf16" else pa.PA_F32
    q, kc, vc, nk, nv = W.make_values(w, dev)
    work = work_split(w)
    pass_bytes = sum(v["bytes"] for v in work.values())
    # cycle enough pool copies that one pass's pages cannot stay in the 256 MB Infinity Cache
    rotate = args.rotate or (1 if pass_bytes >= 8 * MALL_BYTES else int(np.ceil(8 * MALL_BYTES / max(pass_bytes, 1))))
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(max(1, rotate) - 1)]
    rotate = len(pools)

    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    qsl = torch.from_numpy(w.query_start_loc).to(dev)
    slots = None if w.new_slots is None else torch.from_numpy(w.new_slots).to(dev)
    nbytes = pa.pa_forward_workspace_bytes(w.num_seqs, w.num_tokens, w.max_q_len, w.num_q_heads, w.num_kv_heads,
                                           w.head_dim, w.max_context_len, code)
    workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = HipEvents()
    rope = args.workload == "splitfuse_rope"
    if rope:
        # the cache write rotates q (into qrot) and the new keys at their positions first
        ql = np.diff(w.query_start_loc)
        positions = torch.from_numpy(np.concatenate(
            [np.arange(L - n, L) for n, L in zip(ql, w.context_lens)]).astype(np.int32)).to(dev)
        cos_t, sin_t = (torch.from_numpy(t).to(dev) for t in W.rope_tables(w.max_context_len, w.head_dim))
        qrot = torch.empty_like(q)

    def step(i, stage_events=None, write_events=None):
        kcur, vcur = pools[i % rotate]
        qin = q
        if slots is not None:
            if write_events:
                ev.record(write_events[0], stream)
            if rope:
                pa.pa_rope_reshape_and_cache(qrot, q, nk, nv, kcur, vcur, slots, positions, cos_t, sin_t, status)
                qin = qrot
            else:
                pa.pa_reshape_and_cache(nk, nv, kcur, vcur, slots, status)
            if write_events:
                ev.record(write_events[1], stream)
        pa.pa_set_stage_events(stage_events)
        pa.pa_forward(out, qin, kcur, vcur, tables, lens, qsl, w.max_q_len, w.max_context_len, w.scale,
                      workspace, status)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item()):#x}")

    # timed steps: nothing but the path itself on the stream (an event between
    # steps gives each step's device time)
    K = args.steps
    step_ev = ev.new(K + 1)
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        ev.record(step_ev[0], stream)
        for k in range(K):
            step(args.warmup + k)
            ev.record(step_ev[k + 1], stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_ms = np.array([ev.ms(step_ev[k], step_ev[k + 1]) for k in range(K)])

    # the same steps again with HIP events around every stage (kernel durations)
    stage_ev = [ev.new(2 * len(STAGES)) for _ in range(K)]
    write_ev = [ev.new(2) for _ in range(K)] if slots is not None else [None] * K
    for k in range(K):
        step(args.warmup + K + k, stage_ev[k], write_ev[k])
    torch.cuda.synchronize()
    pa.pa_set_stage_events(None)
    stage_all = {name: np.array([ev.ms(e[2 * j], e[2 * j + 1]) for e in stage_ev]) for j, name in enumerate(STAGES)}
    stage_ms = {name: float(np.mean(v)) for name, v in stage_all.items()}
    write_ms = float(np.mean([ev.ms(e[0], e[1]) for e in write_ev])) if slots is not None else 0.0
    ev.close()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item()):#x}")

    ms_per_step = 1e3 * elapsed / K
    # the dominant kernel is the worker with the largest share of the pass: a
    # prefill tile worker is priced against bf16 MFMA, the decode workers against HBM
    dom = max(WORKERS, key=lambda k: stage_ms[k])
    result = {
        "metric": METRIC,
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
    }
    if args.workload in ("splitfuse", "splitfuse_rope"):
        result.update(value=round(w.num_tokens / (ms_per_step * 1e-3), 1), unit="tokens/s")
    else:
        result.update(value=round(pass_bytes / (ms_per_step * 1e-3) / 1e9, 2), unit="GB/s")
    result["step_ms"] = {"median": round(float(np.median(step_ms)), 4), "min": round(float(step_ms.min()), 4),
                         "max": round(float(step_ms.max()), 4), "source": "HIP events between the timed steps"}
    result["config"] = {"workload": w.name, "num_seqs": w.num_seqs, "query_tokens": w.num_tokens,
                        "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                        "block_size": 16, "max_context_len": w.max_context_len, "pool_blocks": w.num_blocks,
                        "pool_copies_rotated": rotate,
                        "kv_residency": ("cold: pool copies cycled past the 256 MB MALL" if rotate > 1 else
                                         "warm: one pool every step, the pass fits the 256 MB MALL"
                                         if pass_bytes <= MALL_BYTES else
                                         f"one pool every step; the pass ({pass_bytes / 1e6:.0f} MB) exceeds "
                                         f"the 256 MB MALL")}
    # a batch of single-position GQA decodes runs in one dispatch of gqa_decode_kernel (the
    # library times it as its MFMA-worker stage)
    G = w.num_q_heads // w.num_kv_heads
    one_pass = w.dtype == "bf16" and w.max_q_len == 1 and 2 <= G <= 16
    dom_kernel = f"gqa_decode_kernel<{w.head_dim}>" if one_pass and dom == "mfma_worker" else \
        DOMINANT_KERNEL[(dom, w.dtype, w.head_dim)]
    traffic = measured_traffic(w.name, dom_kernel)
    if dom == "tile_worker":
        achieved = work[dom]["flops"] / (stage_ms[dom] * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                              "traffic": traffic, "kernel": dom_kernel, "kernel_ms": round(stage_ms[dom], 4),
                              "algorithmic_flops": work[dom]["flops"]}
    else:
        achieved = work[dom]["bytes"] / (stage_ms[dom] * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dom_kernel,
                              "kernel_ms": round(stage_ms[dom], 4), "algorithmic_bytes": work[dom]["bytes"]}
    dk = stage_all[dom]
    result["roofline"]["kernel_ms_median_min_max"] = [round(float(np.median(dk)), 4), round(float(dk.min()), 4),
                                                      round(float(dk.max()), 4)]
    if dom != "tile_worker":
        # the attainable rate for a pure page-read loop over passes of the same size
        probe_gbps, probe_bytes = probe_ceiling(torch, dev, work[dom]["bytes"])
        long_gbps, _ = (probe_gbps, probe_bytes) if probe_bytes >= 4 << 30 else \
            probe_ceiling(torch, dev, 4 << 30)
        result["roofline"]["read_probe"] = {
            "GBps": round(probe_gbps, 1), "pass_bytes": probe_bytes,
            "frac_of_probe": round(result["roofline"]["achieved"] / probe_gbps, 4),
            "GBps_4GiB_pass": round(long_gbps, 1),
            "frac_of_4GiB_probe": round(result["roofline"]["achieved"] / long_gbps, 4),
            "probe": "random 4 KiB pages, non-temporal 16-byte loads, 4 pages per wavefront in flight "
                     "(libpa_probe pa_probe_read_pages), HIP events between back-to-back launches"}
    result["clock"] = clock.summary()
    result["stages_ms"] = {k: round(v, 4) for k, v in stage_ms.items()}
    if slots is not None:
        result["stages_ms"]["rope_cache_write" if rope else "cache_write"] = round(write_ms, 4)
    result["kv_read_GBps"] = round(pass_bytes / (sum(stage_ms[k] for k in WORKERS) * 1e-3) / 1e9, 1)
    for k in ("valu_worker", "mfma_worker"):
        if work[k]["bytes"] and not work[k]["flops"]:
            result[f"{k}_kv_GBps"] = round(work[k]["bytes"] / (stage_ms[k] * 1e-3) / 1e9, 1)
    if work["tile_worker"]["flops"]:
        t_ms = stage_ms["tile_worker"]
        f = work["tile_worker"]["flops"]
        result["prefill"] = {"kernel": "tile_worker", "kernel_ms": round(t_ms, 4),
                             "algorithmic_tflops": round(f / 1e12, 3),
                             "achieved_tflops": round(f / (t_ms * 1e-3) / 1e12, 1),
                             "frac_of_bf16_mfma_peak": round(f / (t_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": measured_traffic(w.name, DOMINANT_KERNEL[("tile_worker", w.dtype,
                                                                                   w.head_dim)])}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, q, kc, vc, args.cpu_seconds)
        mixed = args.workload in ("splitfuse", "splitfuse_rope")
        result["cpu_baseline"] = {
            "value": round(cb["rows"] / cb["seconds"], 3) if mixed else round(cb["kv_bytes"] / cb["seconds"] / 1e9, 4),
            "unit": "tokens/s" if mixed else "GB/s",
            "cores": cb["cores"], "kind": "oracle",
            "sample": f"{cb['rows']} query rows drawn uniformly from the pass's {w.num_tokens} "
                      f"({cb['chunk_rows']} prefill-chunk rows, {cb['rows'] - cb['chunk_rows']} decode rows), each "
                      f"attended at its position by the fp64 oracle (gather + attention over host copies of its "
                      f"sequence's pages): {cb['seconds']:.1f} s of oracle time",
            "host": cb["host"]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

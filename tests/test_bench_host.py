"""Host-side pieces of bench.py: the work each worker is credited with, and the one-GPU guard."""
import subprocess
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_splitfuse_work_split():
    w = bench.build_workload("splitfuse")
    work = bench.work_split(w)
    ql = np.diff(w.query_start_loc)
    L = w.context_lens.astype(np.int64)
    dec = ql == 1
    assert work["valu_worker"]["bytes"] == int(L[dec].sum()) * 2 * 32 * 128 * 2
    assert work["valu_worker"]["flops"] == 0 and work["mfma_worker"] == {"bytes": 0, "flops": 0}
    # causal chunk rows: row i of a chunk of q rows over L keys sees L - q + i + 1 keys
    flops = sum(4 * 128 * 32 * sum(Ls - q + i + 1 for i in range(q)) for q, Ls in zip(ql[~dec], L[~dec]))
    assert work["tile_worker"]["flops"] == flops
    assert work["tile_worker"]["bytes"] == int(L[~dec].sum()) * 2 * 32 * 128 * 2


def test_gqa_decode_goes_to_the_mfma_worker():
    w = bench.build_workload("gqa70b")
    work = bench.work_split(w)
    assert work["mfma_worker"]["bytes"] == 32 * 2048 * 2 * 8 * 128 * 2
    assert work["valu_worker"]["bytes"] == 0 and work["tile_worker"]["bytes"] == 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

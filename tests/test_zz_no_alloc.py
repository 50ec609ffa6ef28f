"""pa_forward_noalloc (workspace in the library's static per-GPU array) against pa_forward
(caller workspace) through the C ABI: two calls in a row, the second on a smaller batch,
each equal to pa_forward bit for bit and to the fp64 oracle within tolerance; a batch
whose workspace exceeds the static array is refused on the host."""
import pytest
import torch

import workloads as W
from tests._gpu import DEV, Run, assert_close, check_tables_in_pool, oracle_rows_all, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_57_amd as pa
    assert torch.cuda.is_available()
    return pa


def run_pair(pa, w, label):
    say(f"[case] no-alloc {label}: S={w.num_seqs} T={w.num_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"maxL={w.max_context_len}")
    check_tables_in_pool(w)
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    ref_out = r.forward(q, kc, vc)
    r.check_status()
    out = torch.full_like(q, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.pa_forward_noalloc(out, q, kc, vc, r.tables, r.lens, r.qsl, w.max_q_len, w.max_context_len, w.scale,
                          status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), label
    rows, ref = oracle_rows_all(w, q, kc, vc)
    assert_close(to_f64(out.index_select(0, torch.from_numpy(rows).to(DEV))), ref, "bf16", f"no-alloc {label}")


def test_noalloc_forward_matches_forward(pa):
    assert pa.pa_forward_noalloc_max_workspace_bytes() == 64 << 20
    # first call: decodes with split contexts, GQA rows and prefill chunks (every worker and the merge)
    big = W.random_ragged(61, "bf16", 16, 4, 128, [1, 1, 300, 1, 40, 1], [4100, 33, 2500, 3000, 700, 1])
    run_pair(pa, big, "first call")
    # second call, smaller: the static workspace keeps the first call's bytes, which must not matter
    small = W.random_ragged(62, "bf16", 8, 8, 128, [1, 20, 1], [600, 20, 1300])
    run_pair(pa, small, "second call, smaller")


def test_noalloc_refuses_batches_beyond_its_workspace(pa):
    w = W.random_ragged(63, "bf16", 32, 32, 128, [1], [40])
    need = pa.pa_forward_workspace_bytes(4096, 4096, 1, 32, 32, 128, 65536, pa.PA_BF16)
    assert need > pa.pa_forward_noalloc_max_workspace_bytes()
    r = Run(w)
    q = torch.zeros((4096, 32, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    ks, vs = W.cache_shapes(w)
    kc = torch.zeros(ks, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(vs, dtype=torch.bfloat16, device=DEV)
    lens = torch.full((4096,), 40, dtype=torch.int32, device=DEV)
    qsl = torch.arange(4097, dtype=torch.int32, device=DEV)
    tables = r.tables.repeat(4096, 1)
    with pytest.raises(pa.PAError) as e:
        pa.pa_forward_noalloc(out, q, kc, vc, tables, lens, qsl, 1, 65536, w.scale)
    assert e.value.status == pa.PA_ERR_INVALID and "static workspace" in str(e.value)

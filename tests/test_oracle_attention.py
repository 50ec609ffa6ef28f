"""Pins of the float64 attention oracle against facts fixed outside it.

Each test names the plausible mistake it would catch.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, layout
from tests._pools import build_case


def run_oracle(c, tokens=None):
    return attention.paged_attention(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], c["qsl"],
                                     c["scale"], c["dtype"], tokens=tokens)


def brute_force(c):
    """Scalar loops with math.exp, straight from softmax(q·k·scale) v over visible keys."""
    qf = layout.to_f64(c["q"], c["dtype"])
    hq, hkv, d = c["hq"], c["hkv"], c["d"]
    G = hq // hkv
    out = np.zeros(qf.shape)
    for s, L in enumerate(c["lens"]):
        a, b = c["qsl"][s], c["qsl"][s + 1]
        K, V = c["Klog"][s], c["Vlog"][s]
        for i in range(b - a):
            pos = L - (b - a) + i
            for h in range(hq):
                g = h // G
                sc = [c["scale"] * sum(qf[a + i, h, e] * K[j, g, e] for e in range(d))
                      for j in range(pos + 1)]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                for e in range(d):
                    out[a + i, h, e] = sum(w[j] * V[j, g, e] for j in range(pos + 1)) / tot
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_tiny_ragged(dtype):
    # catches: wrong query position, off-by-one causal limit, wrong GQA head map,
    # wrong block/offset gather, dropped scale
    c = build_case(3, dtype, hq=4, hkv=2, d=8, lens=[1, 17, 40, 33], qlens=[1, 5, 1, 33])
    np.testing.assert_allclose(run_oracle(c), brute_force(c), rtol=0, atol=1e-12)


def test_single_key_returns_its_value_row():
    # softmax over one key is exactly 1: output must be that value row, bit for bit
    c = build_case(5, "bf16", hq=8, hkv=8, d=64, lens=[1, 1], qlens=[1, 1], scale_q=5.0)
    out = run_oracle(c)
    for s in range(2):
        assert np.array_equal(out[s], c["Vlog"][s][0])


def test_first_row_of_fresh_chunk_sees_one_key():
    # a prefill chunk with no prior context: its first row is causal-limited to key 0
    c = build_case(6, "f32", hq=4, hkv=4, d=16, lens=[20], qlens=[20])
    out = run_oracle(c)
    assert np.array_equal(out[0], c["Vlog"][0][0])


def test_identical_scores_give_mean_of_values():
    # q = 0 makes every score equal: the output is the plain mean of the visible values
    c = build_case(7, "f32", hq=4, hkv=2, d=32, lens=[50, 3], qlens=[4, 1])
    c["q"] = np.zeros_like(c["q"])
    out = run_oracle(c)
    for s, L in enumerate(c["lens"]):
        a, b = c["qsl"][s], c["qsl"][s + 1]
        for i in range(b - a):
            pos = L - (b - a) + i
            want = c["Vlog"][s][:pos + 1].mean(axis=0)           # [Hkv, d]
            got = out[a + i].reshape(c["hkv"], -1, c["d"])        # [Hkv, G, d]
            np.testing.assert_allclose(got, np.repeat(want[:, None], got.shape[1], 1), atol=1e-14, rtol=0)


def _sdpa(q, K, V, scale, mask=None, causal=False, gqa=False):
    from torch.nn.attention import SDPBackend, sdpa_kernel
    with sdpa_kernel(SDPBackend.MATH):
        return torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1)[None], torch.from_numpy(K).transpose(0, 1)[None],
            torch.from_numpy(V).transpose(0, 1)[None], attn_mask=mask, is_causal=causal,
            scale=scale, enable_gqa=gqa)[0].transpose(0, 1).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_matches_torch_sdpa_math_backend(hq, hkv):
    # library special case: a contiguous sequence; fresh causal chunk uses is_causal,
    # a chunk with prior context uses an explicit bottom-right causal mask; GQA uses
    # torch's enable_gqa (query head h reads KV head h // (hq/hkv))
    c = build_case(11, "bf16", hq=hq, hkv=hkv, d=32, lens=[24, 61, 9], qlens=[24, 13, 1])
    out = run_oracle(c)
    qf = layout.to_f64(c["q"], "bf16")
    gqa = hq != hkv
    # sequence 0: prior 0, causal
    ref0 = _sdpa(qf[0:24], c["Klog"][0], c["Vlog"][0], c["scale"], causal=True, gqa=gqa)
    np.testing.assert_allclose(out[0:24], ref0, atol=1e-13, rtol=0)
    # sequence 1: prior 48, chunk of 13
    pos = 48 + np.arange(13)
    mask = torch.from_numpy(np.arange(61)[None, :] <= pos[:, None])
    ref1 = _sdpa(qf[24:37], c["Klog"][1], c["Vlog"][1], c["scale"], mask=mask, gqa=gqa)
    np.testing.assert_allclose(out[24:37], ref1, atol=1e-13, rtol=0)
    # sequence 2: decode row sees all keys
    ref2 = _sdpa(qf[37:38], c["Klog"][2], c["Vlog"][2], c["scale"], gqa=gqa)
    np.testing.assert_allclose(out[37:38], ref2, atol=1e-13, rtol=0)


def test_gqa_equals_mha_with_replicated_kv_heads():
    # catches h % Hkv instead of h // G
    c = build_case(13, "f32", hq=8, hkv=2, d=16, lens=[30, 45], qlens=[3, 1])
    out_gqa = run_oracle(c)
    G = 4
    rep = dict(c)
    x = layout.elems_per_16_bytes("f32")
    rep["kp"] = np.repeat(c["kp"], G, axis=1)
    rep["vp"] = np.repeat(c["vp"], G, axis=1)
    rep["hkv"] = 8
    out_mha = run_oracle(rep)
    assert rep["kp"].shape[1] == 8 and x == 4
    np.testing.assert_allclose(out_gqa, out_mha, atol=1e-13, rtol=0)


def test_invariant_under_physical_block_permutation():
    # moving every physical block and rewriting the tables accordingly changes nothing
    c = build_case(17, "bf16", hq=4, hkv=4, d=64, lens=[100, 37, 16, 1], qlens=[1, 1, 4, 1])
    base = run_oracle(c)
    rng = np.random.default_rng(99)
    nb = c["kp"].shape[0]
    pi = rng.permutation(nb)
    kp2, vp2 = np.empty_like(c["kp"]), np.empty_like(c["vp"])
    kp2[pi] = c["kp"]
    vp2[pi] = c["vp"]
    tab2 = np.where(c["tables"] >= 0, pi[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    moved = dict(c, kp=kp2, vp=vp2, tables=tab2)
    assert np.array_equal(run_oracle(moved), base)


def test_large_scores_stay_finite_and_match_scipy_softmax():
    # q scaled by 8 gives scores of tens of units: max subtraction must keep exp in range
    from scipy.special import softmax
    c = build_case(19, "f32", hq=2, hkv=2, d=64, lens=[300], qlens=[1], scale_q=8.0)
    out = run_oracle(c)
    assert np.isfinite(out).all()
    qf = layout.to_f64(c["q"], "f32")[0]
    K, V = c["Klog"][0], c["Vlog"][0]
    for h in range(2):
        w = softmax(c["scale"] * K[:, h] @ qf[h])
        np.testing.assert_allclose(out[0, h], w @ V[:, h], atol=1e-13, rtol=0)


def test_token_subset_matches_full_output():
    c = build_case(23, "bf16", hq=4, hkv=1, d=32, lens=[70, 20, 5], qlens=[10, 2, 1])
    full = run_oracle(c)
    sub = run_oracle(c, tokens=[12, 0, 9])
    assert np.array_equal(sub, full[[12, 0, 9]])


def test_rejects_more_rows_than_keys():
    c = build_case(29, "f32", hq=2, hkv=2, d=16, lens=[4], qlens=[4])
    c["lens"] = np.array([3], np.int32)
    with pytest.raises(ValueError):
        run_oracle(c)

"""Pins of the tiled online softmax and the log-sum-exp merge against the direct definition."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import online_softmax as osm
from tests.conftest import GOLDEN


def direct(Q, K, V, scale, limits):
    S = scale * (Q @ K.T)
    S = np.where(np.arange(K.shape[0])[None, :] <= np.asarray(limits)[:, None], S, -np.inf)
    W = np.exp(S - S.max(axis=1, keepdims=True))
    return (W @ V) / W.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("br,bc", [(1, 1), (3, 5), (16, 16), (32, 32), (64, 7), (200, 200)])
def test_tiled_equals_direct_fp64(br, bc):
    rng = np.random.default_rng(br * 100 + bc)
    N, L, d = 45, 77, 24
    Q, K, V = (rng.standard_normal((n, d)) for n in (N, L, L))
    lim = rng.integers(0, L, size=N)                 # ragged causal limits
    np.testing.assert_allclose(osm.tiled_attention(Q, K, V, 0.2, br, bc, lim),
                               direct(Q, K, V, 0.2, lim), atol=1e-12, rtol=0)


def test_page_equivalence_check_fp32():
    # "第 15 章：推理引擎与部署" §15.1 Python simulation: seed 42, N=128, d=64,
    # 32x32 tiles, tiled vs standard within atol 1e-5 in float32
    fx = json.load(open(os.path.join(GOLDEN, "online_softmax_check.json")))
    torch.manual_seed(fx["seed"])
    N, d = fx["N"], fx["d"]
    Q, K, V = (torch.randn(N, d).numpy() for _ in range(3))
    scale = np.float32(1.0 / np.sqrt(d))
    tiled = osm.tiled_attention(Q, K, V, scale, fx["block_rows"], fx["block_cols"])
    std = direct(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), float(scale),
                 np.full(N, N - 1))
    assert tiled.dtype == np.float32
    assert np.abs(tiled - std).max() <= fx["atol"]


@pytest.mark.parametrize("part", [1, 16, 17, 100, 512, 10_000])
def test_split_k_merge_equals_direct(part):
    rng = np.random.default_rng(part)
    N, L, d = 9, 700, 16
    Q, K, V = (rng.standard_normal((n, d)) for n in (N, L, L))
    lim = np.array([0, 5, 16, 17, 255, 256, 511, 600, 699])   # some rows see no key of later partitions
    np.testing.assert_allclose(osm.split_k_attention(Q, K, V, 0.3, part, 16, lim),
                               direct(Q, K, V, 0.3, lim), atol=1e-12, rtol=0)


def test_merge_of_empty_partition_is_neutral():
    rng = np.random.default_rng(1)
    Q, K, V = rng.standard_normal((2, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    lim = np.array([10, 19])
    full = osm.partition_state(Q, K, V, 1.0, 0, 20, lim, 16)
    empty = osm.partition_state(Q, K, V, 1.0, 20, 40, lim, 16)
    assert np.isneginf(empty[0]).all() and (empty[1] == 0).all() and (empty[2] == 0).all()
    np.testing.assert_allclose(osm.merge_states([full, empty]), full[2] / full[1], atol=1e-15, rtol=0)


def test_merge_rejects_rows_with_no_keys():
    Q, K, V = np.ones((1, 4)), np.ones((4, 4)), np.ones((4, 4))
    st = osm.partition_state(Q, K, V, 1.0, 0, 4, np.array([-1]), 16)
    with pytest.raises(ValueError):
        osm.merge_states([st])

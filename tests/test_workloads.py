"""Seeded input generators: shapes, distributions and determinism."""
import numpy as np
import pytest

import ep_workloads as W


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_routing_shapes_and_ranges(name):
    sh = W.CONFIGS[name]
    if sh.n_ranks * sh.tokens * sh.hidden > 64 * 1024 * 1024:
        pytest.skip("full-size x is large; routing checked on the smaller configs")
    wl = W.make_workload(sh)
    assert wl.idx.shape == (sh.n_ranks, sh.tokens, sh.topk)
    assert ((wl.idx >= 0) & (wl.idx < sh.n_experts)).all()
    np.testing.assert_allclose(wl.weights.sum(-1), 1.0, rtol=1e-5)


def test_uniform_routing_has_distinct_experts_per_token():
    wl = W.make_workload(W.CONFIGS["tiny"])
    s = np.sort(wl.idx, axis=-1)
    assert (np.diff(s, axis=-1) != 0).all()


def test_rank0_routing_hits_the_bound():
    sh = W.Shape("w", 8, 16, 64, 48, 8, routing="rank0")     # L = 6 < R = 8
    wl = W.make_workload(sh)
    assert (wl.idx // (sh.n_experts // sh.n_ranks) == 0).all()
    assert (wl.idx[..., :6].max(-1) < 6).all()


def test_generator_is_deterministic():
    a = W.make_workload(W.CONFIGS["tiny_zipf"])
    b = W.make_workload(W.CONFIGS["tiny_zipf"])
    for x, y in ((a.idx, b.idx), (a.weights, b.weights), (a.x_bf16, b.x_bf16)):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name", sorted(W.KV_CONFIGS))
def test_kv_tables_are_distinct_pool_blocks(name):
    sh = W.KV_CONFIGS[name]
    src, dst = W.make_kv_tables(sh)
    assert len(src) == -(-sh.tokens // sh.src_block_tokens)
    assert len(dst) == -(-sh.tokens // sh.dst_block_tokens)
    for t, pool in ((src, sh.src_pool_blocks), (dst, sh.dst_pool_blocks)):
        assert len(np.unique(t)) == len(t)
        assert t.min() >= 0 and t.max() < pool


def test_kv_free_list_runs_have_the_requested_mean():
    sh = W.KvShape("m", 1, 100000, 16, 1, 1, 200000, 200000, 40.0, 40.0, seed=1)
    src, _ = W.make_kv_tables(sh)
    runs = 1 + int((np.diff(src) != 1).sum())
    assert 30 < len(src) / runs < 55

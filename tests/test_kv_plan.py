"""Host-side KV region planner of the library against the oracle (CPU)."""
import numpy as np
import pytest

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle


@pytest.mark.parametrize("bs_src,bs_dst,run_s,run_d,seed", [
    (1, 1, 8.0, 3.0, 0), (4, 16, 2.0, 5.0, 1), (16, 4, 1.0, 1.0, 2), (3, 5, 4.0, 2.0, 3),
    (64, 64, 2.0, 2.0, 4), (1, 16, 1000.0, 1000.0, 5)])
def test_kv_plan_merged_equals_oracle(bs_src, bs_dst, run_s, run_d, seed):
    sh = W.KvShape("t", 2, 301, 48, bs_src, bs_dst, 400, 400, run_s, run_d, seed)
    src, dst = W.make_kv_tables(sh)
    got = ep.kv_plan(sh.tokens, sh.token_bytes, bs_src, src, bs_dst, dst)
    want = oracle.kv_regions(sh.tokens, sh.token_bytes, bs_src, src, bs_dst, dst)
    np.testing.assert_array_equal(got[:, :3], want)
    np.testing.assert_array_equal(got[:, 3], np.concatenate([[0], np.cumsum(want[:, 2])[:-1]]))


def test_kv_plan_unmerged_pieces_stay_in_blocks():
    sh = W.KvShape("t", 2, 301, 48, 4, 6, 400, 400, 50.0, 50.0, 7)
    src, dst = W.make_kv_tables(sh)
    raw = ep.kv_plan(sh.tokens, 48, 4, src, 6, dst, merge=False)
    merged = ep.kv_plan(sh.tokens, 48, 4, src, 6, dst)
    assert raw[:, 2].sum() == merged[:, 2].sum() == 301 * 48
    assert len(raw) >= len(merged)
    # every piece lies inside one source block and one destination block
    for so, do, by, _ in raw:
        assert so // (4 * 48) == (so + by - 1) // (4 * 48)
        assert do // (6 * 48) == (do + by - 1) // (6 * 48)
    # applying either list moves the same bytes
    rng = np.random.default_rng(0)
    s = rng.integers(0, 256, size=(1, 400 * 4 * 48), dtype=np.uint8)
    d = np.zeros((1, 400 * 6 * 48), np.uint8)
    np.testing.assert_array_equal(oracle.kv_copy(raw[:, :3], s, d), oracle.kv_copy(merged[:, :3], s, d))


def test_kv_plan_rejects_bad_arguments():
    for args in [(10, 24, 1, [0] * 10, 1, [0] * 10),     # token bytes not a multiple of 16
                 (10, 16, 0, [0] * 10, 1, [0] * 10),     # block size 0
                 (2, 16, 1, [0, -1], 1, [0, 1])]:         # negative block id
        with pytest.raises(ep.EPError) as e:
            ep.kv_plan(*args)
        assert e.value.code == ep.EP_ERR_INVALID_ARG
    assert ep.kv_plan(0, 16, 1, [], 1, []).shape == (0, 4)

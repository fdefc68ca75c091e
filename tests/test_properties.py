"""Property-based checks (hypothesis, CPU): the library's host-side KV
planner against the oracle, and the oracle's plan against its defining
invariants, on random small inputs."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import combine_ep_plan_amd as ep
import oracle

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def kv_case(draw):
    n = draw(st.integers(0, 200))
    tok = 16 * draw(st.integers(1, 8))
    bs_src = draw(st.integers(1, 9))
    bs_dst = draw(st.integers(1, 9))
    ns, nd = -(-n // bs_src), -(-n // bs_dst)
    pool_s = ns + draw(st.integers(0, 20))
    pool_d = nd + draw(st.integers(0, 20))
    src = draw(st.permutations(list(range(pool_s))))[:ns]
    dst = draw(st.permutations(list(range(pool_d))))[:nd]
    return n, tok, bs_src, np.array(src, np.int32), bs_dst, np.array(dst, np.int32)


@SETTINGS
@given(kv_case())
def test_kv_planner_matches_oracle(case):
    n, tok, bs_src, src, bs_dst, dst = case
    got = ep.kv_plan(n, tok, bs_src, src, bs_dst, dst)
    want = oracle.kv_regions(n, tok, bs_src, src, bs_dst, dst)
    np.testing.assert_array_equal(got[:, :3], want)
    if len(want):
        np.testing.assert_array_equal(got[:, 3], np.concatenate([[0], np.cumsum(want[:, 2])[:-1]]))
    raw = ep.kv_plan(n, tok, bs_src, src, bs_dst, dst, merge=False)
    assert raw[:, 2].sum() == n * tok and len(raw) >= len(want)


@st.composite
def routing(draw):
    N = draw(st.integers(1, 6))
    L = draw(st.integers(1, 5))
    E = N * L
    T = draw(st.integers(0, 12))
    R = draw(st.integers(1, 6))
    idx = draw(st.lists(st.integers(-1, E), min_size=N * T * R, max_size=N * T * R))
    return N, T, E, R, np.array(idx, np.int32).reshape(N, T, R)


@SETTINGS
@given(routing())
def test_oracle_plan_invariants(case):
    N, T, E, R, idx = case
    L = E // N
    cap = oracle.recv_bound(N, T, E, R)
    p = oracle.plan(N, T, E, R, cap, idx)
    valid = (idx >= 0) & (idx < E)
    assert (p["status"] & oracle.STATUS_BAD_EXPERT != 0) == bool((~valid).any())
    # counts: a histogram of the valid ids per source
    for s in range(N):
        np.testing.assert_array_equal(p["cnt"][s], np.bincount(idx[s][valid[s]], minlength=E))
    # send positions: a permutation of [0, valid count) per source, ordered by (expert, t, k)
    for s in range(N):
        sp = p["send_pos"][s][valid[s]]
        assert sorted(sp.tolist()) == list(range(int(valid[s].sum())))
        keys = [(int(e), t, k) for t in range(T) for k in range(R)
                for e in [idx[s, t, k]] if 0 <= e < E]
        order = sorted(range(len(keys)), key=lambda i: keys[i])
        np.testing.assert_array_equal(np.argsort(sp, kind="stable"), order)
    assert (p["send_pos"][~valid] == -1).all()
    # grouped positions: a bijection onto [0, total_d) per destination
    totals = p["recv_off"][:, N]
    for d in range(N):
        mine = valid & (idx // L == d) if L else valid
        gp = p["grp_pos"][mine]
        assert sorted(gp.tolist()) == list(range(int(totals[d])))
    assert int(totals.sum()) == int(valid.sum())

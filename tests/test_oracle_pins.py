"""Pins for the CPU oracle, independent of the oracle's own code.

Each check ties the oracle to something it does not compute itself: a
library routine (numpy's stable argsort, torch's number-format casts), a
brute force written here in plain Python, a closed form, an invariant, a
hand-worked example, or the receive bound printed in "Enabling
trillion-parameter models on AWS EFA", section "Send and receive buffers".
"""
import bisect
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import ep_workloads as W
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Brute-force helpers written independently of the oracle
# ---------------------------------------------------------------------------

def _all_finite_bf16():
    """Every finite bf16 value as (exact Fraction, bit pattern), sorted."""
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    vals = ((bits << 16).astype(np.uint32)).view(np.float32)
    out = {}
    for b, v in zip(bits.tolist(), vals.tolist()):
        if np.isfinite(v):
            fr = Fraction(v)
            # keep +0 for zero, the even pattern wins ties below anyway
            if fr not in out or (b & 0x8000) == 0:
                out[fr] = b
    keys = sorted(out)
    return keys, [out[k] for k in keys]


_BF16_TABLE = None


def brute_bf16_round(x: Fraction) -> int:
    """Nearest bf16 to an exact rational, ties to the even pattern."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = _all_finite_bf16()
    keys, bits = _BF16_TABLE
    if x == 0:
        return 0
    if x < 0:                       # round the magnitude, keep the sign (-0)
        return 0x8000 | brute_bf16_round(-x)
    i = bisect.bisect_left(keys, x)
    if i < len(keys) and keys[i] == x:
        return bits[i]
    lo, hi = keys[i - 1], keys[i]
    dlo, dhi = x - lo, hi - x
    if dlo < dhi:
        return bits[i - 1]
    if dhi < dlo:
        return bits[i]
    return bits[i - 1] if bits[i - 1] % 2 == 0 else bits[i]


def bf16_value(b: int) -> Fraction:
    return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))


def brute_plan(idx, N, T, E, R, cap):
    """Layout by sorting tuples, one destination at a time (plain Python)."""
    L = E // N
    send_pos = np.full((N, T, R), -1, np.int64)
    for s in range(N):
        slots = [(int(idx[s, t, k]), t, k) for t in range(T) for k in range(R)
                 if 0 <= idx[s, t, k] < E]
        for p, (_, t, k) in enumerate(sorted(slots)):
            send_pos[s, t, k] = p
    grp_pos = np.full((N, T, R), -1, np.int64)
    totals = []
    for d in range(N):
        mine = [(int(idx[s, t, k]) - d * L, s, t, k)
                for s in range(N) for t in range(T) for k in range(R)
                if 0 <= idx[s, t, k] < E and idx[s, t, k] // L == d]
        for p, (_, s, t, k) in enumerate(sorted(mine)):
            grp_pos[s, t, k] = p if p < cap else -1
        totals.append(len(mine))
    return send_pos, grp_pos, totals


def random_idx(rng, N, T, E, R, distinct=True):
    if distinct:
        return np.argsort(rng.random((N, T, E)), axis=-1)[..., :R].astype(np.int32)
    return rng.integers(0, E, size=(N, T, R), dtype=np.int32)


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_rounding_mode():
    assert oracle.lib().oracle_rounding_mode_is_nearest() == 1


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormal
        (rng.standard_normal(2000) * 1e38).astype(np.float32),    # near max
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1.00390625,
                  1.01171875, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
    ])
    # every representable tie in one binade: 1 + (2m+1) * 2^-8
    vals = np.concatenate([vals, (1.0 + (2 * np.arange(128) + 1) * 2.0 ** -8).astype(np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_f64_to_bf16_matches_brute_force():
    """Single rounding from double, checked against the nearest of all bf16."""
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(3000) * 10.0)
    vals += list(rng.standard_normal(300) * 1e-39)
    # double-rounding traps: a float cast first would round these to a tie
    vals += [1.0 + 2 ** -8 + 2 ** -30, 1.0 + 2 ** -8 - 2 ** -30,
             -(1.0 + 2 ** -8 + 2 ** -40), 3.0 + 2 ** -7 + 2 ** -35]
    for v in vals:
        assert oracle.f64_to_bf16(v) == brute_bf16_round(Fraction(v)), v
    # 1 + 2^-8 + 2^-30 lies above the tie between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even


def test_bf16_to_f32_exact():
    for b in [0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x4049]:
        assert oracle.bf16_to_f32(b) == float(np.array([b << 16], np.uint32).view(np.float32)[0])


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(want)
    assert nan.sum() == 2                       # S.1111.111 only
    assert np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ---------------------------------------------------------------------------
# Receive bound (printed formula)
# ---------------------------------------------------------------------------

def test_recv_bound_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "recv_bound.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 5
    for name, N, T, E, R, bound in rows:
        assert oracle.recv_bound(int(N), int(T), int(E), int(R)) == int(bound), name


# ---------------------------------------------------------------------------
# Plan
# ---------------------------------------------------------------------------

HAND_IDX = np.array([[[1, 2], [0, 1]], [[3, 1], [1, 0]]], np.int32)


def test_plan_hand_worked_example():
    """N=2, T=2, E=4, R=2 (L=2), worked out by hand from the definitions."""
    p = oracle.plan(2, 2, 4, 2, 8, HAND_IDX)
    assert p["status"] == 0
    np.testing.assert_array_equal(p["cnt"], [[1, 2, 1, 0], [1, 2, 0, 1]])
    np.testing.assert_array_equal(p["send_off"], [[0, 1, 3, 4, 4], [0, 1, 3, 3, 4]])
    np.testing.assert_array_equal(p["send_pos"], [[[1, 3], [0, 2]], [[3, 1], [2, 0]]])
    np.testing.assert_array_equal(p["recv_off"], [[0, 3, 6], [0, 1, 2]])
    np.testing.assert_array_equal(p["grp_off"], [[0, 2, 6], [0, 1, 2]])
    np.testing.assert_array_equal(p["grp_pos"], [[[2, 0], [0, 3]], [[1, 4], [5, 1]]])


def test_payload_hand_worked_example():
    """Token rows tagged by (s, t); send, receive and grouped rows by hand."""
    sh = W.Shape("hand", 2, 2, 8, 4, 2)
    wl = W.make_workload(sh, idx=HAND_IDX)
    tag = np.zeros((2, 2, 16), np.uint8)
    for s in range(2):
        for t in range(2):
            tag[s, t, :] = 10 * s + t + 1           # x_st tagged as 10s+t+1
    wl.planes = [tag]
    r = oracle.run(wl, cap=8)
    first = lambda a: a[..., 0].tolist()
    # x00=1, x01=2, x10=11, x11=12
    assert first(r["send"][0]) == [[2, 1, 2, 1], [12, 11, 12, 11]]
    assert first(r["recv"][0])[0] == [2, 1, 2, 12, 11, 12]
    assert first(r["recv"][0])[1][:2] == [1, 11]
    assert first(r["grouped"][0])[0] == [2, 12, 1, 2, 11, 12]
    assert first(r["grouped"][0])[1][:2] == [1, 11]


@pytest.mark.parametrize("N,T,E,R,distinct,seed", [
    (4, 16, 16, 2, True, 0), (3, 7, 9, 3, True, 1), (1, 9, 5, 2, True, 2),
    (5, 4, 5, 1, True, 3), (2, 6, 8, 4, False, 4), (6, 3, 12, 5, False, 5),
])
def test_plan_matches_brute_force(N, T, E, R, distinct, seed):
    rng = np.random.default_rng(seed)
    idx = random_idx(rng, N, T, E, R, distinct)
    cap = oracle.recv_bound(N, T, E, R)
    p = oracle.plan(N, T, E, R, cap, idx)
    sp, gp, totals = brute_plan(idx, N, T, E, R, cap)
    np.testing.assert_array_equal(p["send_pos"], sp)
    np.testing.assert_array_equal(p["grp_pos"], gp)
    np.testing.assert_array_equal(p["recv_off"][:, N], totals)
    assert p["status"] == 0


@pytest.mark.parametrize("name", ["tiny", "tiny_zipf", "decode", "worst"])
def test_plan_matches_stable_argsort(name):
    """Send order of a source is numpy's stable argsort of its expert ids."""
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    L = E // N
    p = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), wl.idx)
    assert p["status"] == 0
    for s in range(N):
        flat = wl.idx[s].ravel()
        order = np.argsort(flat, kind="stable")
        inv = np.empty_like(order)
        inv[order] = np.arange(order.size)
        np.testing.assert_array_equal(p["send_pos"][s].ravel(), inv)
        np.testing.assert_array_equal(p["cnt"][s], np.bincount(flat, minlength=E))
    # grouped order of destination d: stable argsort of (local expert) over
    # the slot stream of all sources in (s, t, k) order, restricted to d.
    allflat = wl.idx.reshape(-1)
    gpf = p["grp_pos"].reshape(-1)
    for d in range(N):
        sel = np.nonzero(allflat // L == d)[0]
        order = sel[np.argsort(allflat[sel] - d * L, kind="stable")]
        np.testing.assert_array_equal(gpf[order], np.arange(order.size))


@pytest.mark.parametrize("name", ["tiny", "tiny_zipf", "decode", "worst", "decode_zipf"])
def test_plan_invariants(name):
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    L = E // N
    bound = oracle.recv_bound(N, T, E, R)
    p = oracle.plan(N, T, E, R, bound, wl.idx)
    assert (p["cnt"].sum(axis=1) == T * R).all()
    rows = np.array([[p["send_off"][s, (d + 1) * L] - p["send_off"][s, d * L]
                      for d in range(N)] for s in range(N)])
    assert (rows.sum(axis=1) == T * R).all()            # per-destination counts
    for s in range(N):
        assert sorted(p["send_pos"][s].ravel().tolist()) == list(range(T * R))
    totals = p["recv_off"][:, N]
    assert totals.sum() == N * T * R
    assert (totals <= bound).all()
    np.testing.assert_array_equal(p["grp_off"][:, L], totals)
    d_of = wl.idx // L
    for d in range(N):
        g = np.sort(p["grp_pos"][d_of == d])
        np.testing.assert_array_equal(g, np.arange(totals[d]))
    if name == "worst":
        assert totals[0] == bound and (totals[1:] == 0).all()


def test_plan_single_rank_grouped_equals_send():
    rng = np.random.default_rng(7)
    idx = random_idx(rng, 1, 33, 6, 3)
    p = oracle.plan(1, 33, 6, 3, oracle.recv_bound(1, 33, 6, 3), idx)
    np.testing.assert_array_equal(p["grp_pos"], p["send_pos"])
    np.testing.assert_array_equal(p["recv_off"], [[0, 99]])


def test_plan_topk1_is_counting_sort():
    rng = np.random.default_rng(8)
    N, T, E = 4, 50, 8
    idx = rng.integers(0, E, size=(N, T, 1), dtype=np.int32)
    p = oracle.plan(N, T, E, 1, oracle.recv_bound(N, T, E, 1), idx)
    for s in range(N):
        order = np.argsort(idx[s, :, 0], kind="stable")
        np.testing.assert_array_equal(p["send_pos"][s, order, 0], np.arange(T))


def test_plan_bad_expert_and_capacity():
    idx = HAND_IDX.copy()
    idx[0, 0, 1] = 4          # out of range
    idx[1, 1, 0] = -1         # out of range
    p = oracle.plan(2, 2, 4, 2, 8, idx)
    assert p["status"] == oracle.STATUS_BAD_EXPERT
    assert p["send_pos"][0, 0, 1] == -1 and p["grp_pos"][1, 1, 0] == -1
    assert p["cnt"].sum() == 6
    # capacity 4: destination 0 needs 5 rows now, row 4 is dropped
    p = oracle.plan(2, 2, 4, 2, 4, idx)
    assert p["status"] == oracle.STATUS_BAD_EXPERT | oracle.STATUS_CAPACITY
    assert (p["grp_pos"] < 4).all()
    assert (p["grp_pos"] == -1).sum() == 3
    assert p["recv_off"][0, 2] == 5


# ---------------------------------------------------------------------------
# Payload and combine
# ---------------------------------------------------------------------------

def _src_of_grouped(p, idx, N, E):
    L = E // N
    src = {}
    for s, t, k in np.ndindex(idx.shape):
        g = p["grp_pos"][s, t, k]
        if g >= 0:
            src[(int(idx[s, t, k]) // L, int(g))] = (s, t)
    return src


@pytest.mark.parametrize("name", ["tiny", "tiny_zipf"])
def test_grouped_rows_are_source_rows(name):
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    r = oracle.run(wl)
    p = r["plan"]
    src = _src_of_grouped(p, wl.idx, sh.n_ranks, sh.n_experts)
    assert len(src) == sh.n_ranks * sh.tokens * sh.topk
    for (d, g), (s, t) in src.items():
        np.testing.assert_array_equal(r["grouped"][0][d, g], wl.planes[0][s, t])
    for s in range(sh.n_ranks):   # send rows are x rows, per send_pos
        for t, k in np.ndindex(sh.tokens, sh.topk):
            np.testing.assert_array_equal(r["send"][0][s, p["send_pos"][s, t, k]],
                                          wl.planes[0][s, t])


def test_staged_overflow_rows_are_source_rows_or_zeros():
    """A receive buffer of cap rows keeps the first cap rows of each
    destination in receive order (source rank, then segment row); the
    grouped rows below cap are the x rows their slots name (by a brute-force
    walk of the receive order) when the slot's receive row fitted, else
    zeros. Rows the unpack does not own keep the fill byte."""
    # Rank 0 receives 18 rows: sources 0 and 1 send to its expert 1, source 2
    # to its expert 0. With cap 16 the receive buffer loses source 2's last
    # two rows, which the grouped order puts first (expert 0): rows 4 and 5
    # must be zeros, while grouped rows 16 and 17 fall past cap.
    sh = W.Shape("staged_tight", 3, 6, 16, 6, 2, seed=14)
    idx = np.zeros((3, 6, 2), np.int32)
    idx[0] = [1, 2]
    idx[1] = [1, 4]
    idx[2] = [0, 5]
    wl = W.make_workload(sh, idx=idx)
    cap = 16
    p = oracle.plan(3, 6, 6, 2, cap, wl.idx)
    send = oracle.dispatch_pack(wl.planes[0], p)
    recv = oracle.transfer(send, p, cap)
    grouped = oracle.unpack(recv, p, cap, fill=0xAB)
    x = wl.planes[0]
    for d in range(3):
        # receive order: for each source, its slots for rank d in (expert, t, k) order
        order = []
        for s in range(3):
            order += sorted((int(wl.idx[s, t, k]), t, k, s) for t in range(6) for k in range(2)
                            if wl.idx[s, t, k] // 2 == d)
        grp = sorted(order, key=lambda q: (q[0], q[3], q[1], q[2]))
        fitted = {q for i, q in enumerate(order) if i < cap}
        for r in range(cap):
            if r >= len(grp):
                assert (grouped[d, r] == 0xAB).all()
                continue
            e, t, k, s = grp[r]
            want = x[s, t] if (e, t, k, s) in fitted else np.zeros_like(x[s, t])
            np.testing.assert_array_equal(grouped[d, r], want, err_msg=f"{d} {r}")
    assert p["status"] & oracle.STATUS_CAPACITY
    assert (grouped[0, 4:6] == 0).all() and (grouped[0, :4] != 0).any(axis=1).all()


@pytest.mark.parametrize("name", ["tiny", "tiny_zipf"])
def test_combine_identity_closed_form(name):
    """Identity experts and weights summing to one give back x exactly."""
    wl = W.make_workload(W.CONFIGS[name])
    r = oracle.run(wl)
    np.testing.assert_array_equal(r["out"], wl.x_bf16)


def test_combine_identity_repeated_ids():
    """All slots on rank 0 with repeated expert ids: still x exactly."""
    sh = W.Shape("mini_worst", 8, 8, 64, 32, 8, routing="rank0")
    wl = W.make_workload(sh)
    r = oracle.run(wl)
    assert r["plan"]["recv_off"][0, 8] == oracle.recv_bound(8, 8, 32, 8)
    np.testing.assert_array_equal(r["out"], wl.x_bf16)


def _np_expert_scale(x_bits, a):
    """bf16(x * a) with a float32 multiply (numpy) and torch's bf16 cast."""
    prod = W.bf16_bits_to_f32(x_bits) * np.float32(a)
    return torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_combine_exact_brute_force_scale_expert():
    """Exact rational weighted sum, nearest bf16 by search, no layout."""
    sh = W.Shape("small_scale", 4, 6, 16, 8, 3, expert="scale", seed=3)
    wl = W.make_workload(sh)
    r = oracle.run(wl)
    for s, t in np.ndindex(sh.n_ranks, sh.tokens):
        ys = [_np_expert_scale(wl.x_bf16[s, t], wl.alpha[e]) for e in wl.idx[s, t]]
        for h in range(sh.hidden):
            acc = sum(Fraction(float(wl.weights[s, t, k])) * bf16_value(int(ys[k][h]))
                      for k in range(sh.topk))
            assert r["out"][s, t, h] == brute_bf16_round(acc), (s, t, h)


def test_combine_scale_expert_approx_closed_form():
    """out ~= x * sum_k w_k alpha_k within two bf16 roundings."""
    sh = W.Shape("mid_scale", 8, 32, 512, 64, 8, expert="scale", seed=5)
    wl = W.make_workload(sh)
    r = oracle.run(wl)
    x = W.bf16_bits_to_f32(wl.x_bf16).astype(np.float64)
    f = (wl.weights.astype(np.float64) * wl.alpha[wl.idx].astype(np.float64)).sum(-1)
    want = x * f[..., None]
    got = W.bf16_bits_to_f32(r["out"]).astype(np.float64)
    nz = want != 0
    rel = np.abs(got[nz] - want[nz]) / np.abs(want[nz])
    assert rel.max() <= 2 * 2.0 ** -8


def test_expert_dequant_matches_torch():
    sh = W.Shape("small_fp8", 2, 4, 512, 8, 2, payload=W.PAYLOAD_FP8_B128,
                 expert="dequant", seed=6)
    wl = W.make_workload(sh)
    codes, scales = wl.planes[0], wl.planes[1].view(np.float32)
    for s, t in np.ndindex(2, 4):
        got = oracle.expert_row([codes[s, t], wl.planes[1][s, t]], 0, 1, 512, None)
        deq = torch.from_numpy(codes[s, t].copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        prod = deq * np.repeat(scales[s, t], 128)
        want = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(got, want)
    # dequantised rows stay within the e4m3 half-ulp of the bf16 input
    r = oracle.run(wl)
    x = W.bf16_bits_to_f32(wl.x_bf16)
    y = W.bf16_bits_to_f32(r["out"])
    big = np.abs(x) > 0.05 * np.abs(x).max()
    assert (np.abs(y - x)[big] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(x)[big] + 1e-30).all()


def test_combine_token_rounds_once():
    """Exact sum 1 + 2^-8 + 2^-30 sits just above a bf16 tie: a single
    rounding of the exact sum gives 1 + 2^-7; rounding a float partial sum
    first would land on the tie and give 1."""
    one = np.array([0x3F80], np.uint16)
    w = np.array([1.0 + 2.0 ** -8, 2.0 ** -30], np.float32)
    assert oracle.combine_token(w, [one, one])[0] == 0x3F81
    w = np.array([1.0 + 2.0 ** -8, -(2.0 ** -30)], np.float32)
    assert oracle.combine_token(w, [one, one])[0] == 0x3F80
    w = np.array([0.25, 0.75], np.float32)               # dropped slot skipped
    assert oracle.combine_token(w, [None, one])[0] == 0x3F40


def test_combine_skips_dropped_slots():
    sh = W.Shape("drop", 2, 2, 8, 4, 2)
    idx = HAND_IDX.copy()
    idx[0, 0, 1] = 9
    wl = W.make_workload(sh, idx=idx)
    r = oracle.run(wl, cap=8)
    w = wl.weights[0, 0, 0]
    x = W.bf16_bits_to_f32(wl.x_bf16[0, 0]).astype(np.float64)
    want = np.array([brute_bf16_round(Fraction(float(w)) * Fraction(float(v))) for v in x])
    np.testing.assert_array_equal(r["out"][0, 0], want)


# ---------------------------------------------------------------------------
# Block-fp8 quantisation (sender-side fp8 dispatch)
# ---------------------------------------------------------------------------

def _all_e4m3_values():
    codes = np.arange(0x7F, dtype=np.uint8)                  # non-negative finite
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_f32_to_e4m3_matches_torch_including_ties():
    vals = _all_e4m3_values().astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2                        # exact ties
    eps = np.nextafter(mids.astype(np.float32), np.float32(np.inf)) - mids.astype(np.float32)
    rng = np.random.default_rng(9)
    probe = np.concatenate([
        vals, mids, mids + 1e-7 * mids, mids - 1e-7 * mids,
        rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 5000) * 2.0 ** -6,
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10],
    ]).astype(np.float32)
    probe = np.concatenate([probe, -probe])
    want = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in probe], np.uint8)
    np.testing.assert_array_equal(got, want)
    assert oracle.f32_to_e4m3(1000.0) == 0x7E and oracle.f32_to_e4m3(-1e9) == 0xFE   # saturate
    assert oracle.f32_to_e4m3(2.0 ** -10) == 0x00 and oracle.f32_to_e4m3(3 * 2.0 ** -10) == 0x02


def test_quantize_b128_matches_generator_quantiser():
    """The oracle's quantiser (search encoder) against the workload
    generator's (torch cast), on random rows and hand-made edge blocks."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((6, 512)) * rng.choice([1e-3, 1.0, 40.0], size=(6, 1))).astype(np.float32)
    x[0, :128] = 0.0                                         # all-zero block: scale 1
    x[1, 128:256] = 0.0
    x[1, 200] = -3.0                                         # one non-zero value
    x[2, 256:384] = -0.0                                     # negative zeros
    xb = W.to_bf16_bits(x)
    codes, scales = oracle.quantize_b128(xb)
    gc, gs = W.quantize_fp8_b128(xb)
    np.testing.assert_array_equal(scales, gs)
    np.testing.assert_array_equal(codes, gc)
    assert scales[0, 0] == 1.0 and (codes[0, :128] == 0).all()
    assert codes[1, 200] == 0xFE                             # -448 after scaling by 3/448
    assert (codes[2, 256:384] == 0x80).all()                 # -0 keeps its sign


def test_quantize_b128_roundtrip_error_bound():
    """Dequantised values stay within half an e4m3 ulp (2^-4 relative) of x
    for normal codes, and within half the smallest subnormal step below."""
    rng = np.random.default_rng(11)
    xb = W.to_bf16_bits(rng.standard_normal((4, 1024)).astype(np.float32))
    codes, scales = oracle.quantize_b128(xb)
    x = W.bf16_bits_to_f32(xb).astype(np.float64)
    deq = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    deq *= np.repeat(scales.astype(np.float64), 128, axis=-1)
    q = np.abs(x) / np.repeat(scales.astype(np.float64), 128, axis=-1)
    normal = q >= 2.0 ** -6
    assert (np.abs(deq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6)).all()
    sub = ~normal
    assert (np.abs(deq - x)[sub] <= 2.0 ** -10 * np.repeat(scales, 128, axis=-1)[sub] * (1 + 1e-6)).all()


def test_f32_to_e4m3_saturates_infinities():
    """e4m3fn has no infinity; like any magnitude past 448 it saturates."""
    assert oracle.f32_to_e4m3(float("inf")) == 0x7E
    assert oracle.f32_to_e4m3(float("-inf")) == 0xFE
    assert oracle.f32_to_e4m3(float("nan")) == 0x7F
    assert oracle.f32_to_e4m3(-float("nan")) == 0x7F


BF16_NAN, BF16_NEG_NAN, BF16_SNAN, BF16_INF, BF16_NEG_INF = 0x7FC0, 0xFFC1, 0x7F81, 0x7F80, 0xFF80


def test_quantize_b128_non_finite_blocks():
    """NaN is left out of amax and codes 0x7F; an infinite value makes its
    block's scale infinite, codes itself 0x7F and zeroes the block's finite
    values (signed). Finite blocks beside them are untouched: they equal the
    torch-cast quantiser of the workload generator."""
    rng = np.random.default_rng(12)
    xb = W.to_bf16_bits(rng.standard_normal((4, 512)).astype(np.float32))
    clean = xb.copy()
    xb[0, 3] = BF16_NAN
    xb[0, 200] = BF16_NEG_NAN
    xb[0, 300] = BF16_SNAN
    xb[1, 130] = BF16_INF
    xb[2, 511] = BF16_NEG_INF
    xb[3, 0:128] = BF16_NAN                         # an all-NaN block: amax 0, scale 1
    codes, scales = oracle.quantize_b128(xb)
    # NaN positions and the infinities themselves
    for r, c in [(0, 3), (0, 200), (0, 300), (1, 130), (2, 511)]:
        assert codes[r, c] == 0x7F, (r, c)
    assert (codes[3, :128] == 0x7F).all() and scales[3, 0] == 1.0
    # NaN blocks: amax of the finite values, as if the NaN were a zero
    no_nan = clean.copy()
    no_nan[0, [3, 200, 300]] = 0
    gc, gs = W.quantize_fp8_b128(no_nan)
    keep = np.ones(512, bool)
    keep[[3, 200, 300]] = False
    np.testing.assert_array_equal(codes[0, keep], gc[0, keep])
    np.testing.assert_array_equal(scales[0], gs[0])
    # infinite blocks: scale inf, finite values to +-0 by sign
    assert np.isinf(scales[1, 1]) and np.isinf(scales[2, 3])
    for r, blk, skip in [(1, 1, 130), (2, 3, 511)]:
        lo = 128 * blk
        idx = [i for i in range(lo, lo + 128) if i != skip]
        want = np.where(xb[r, idx] & 0x8000, 0x80, 0x00)
        np.testing.assert_array_equal(codes[r, idx], want)
    # the other blocks of those rows are the plain quantiser's
    gc, gs = W.quantize_fp8_b128(clean)
    for r, blk in [(1, 0), (1, 2), (1, 3), (2, 0), (2, 1), (2, 2)]:
        sl = slice(128 * blk, 128 * blk + 128)
        np.testing.assert_array_equal(codes[r, sl], gc[r, sl])
        assert scales[r, blk] == gs[r, blk]


def _send_rows_by_argsort(idx, E):
    """(source, send row) -> token of that row, from numpy's stable argsort
    of each source's expert ids (valid ids only), independent of the plan."""
    N, T, R = idx.shape
    out = {}
    for s in range(N):
        flat = idx[s].reshape(-1)
        ok = np.nonzero((flat >= 0) & (flat < E))[0]
        order = ok[np.argsort(flat[ok], kind="stable")]
        for p, slot in enumerate(order):
            out[(s, p)] = slot // R
    return out


def test_dispatch_pack_quant_is_quantise_then_place():
    """The fused sender's planes: every send row p of source s holds the
    torch-cast quantisation of the token that the stable argsort puts at p;
    rows past the valid slots stay zero. Repeated and out-of-range ids."""
    sh = W.Shape("pq", 3, 9, 384, 12, 3, payload=W.PAYLOAD_FP8_B128, expert="dequant", seed=13)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    idx[0, 2, 1] = idx[0, 2, 0]                      # repeated id within a token
    idx[1, 4, 2] = 12                                # out of range: dropped
    idx[2, 8, 0] = -1
    p = oracle.plan(3, 9, 12, 3, oracle.recv_bound(3, 9, 12, 3), idx)
    codes, scales = oracle.dispatch_pack_quant(wl.x_bf16, p)
    gc, gs = W.quantize_fp8_b128(wl.x_bf16)
    rows = _send_rows_by_argsort(idx, 12)
    want_c = np.zeros_like(codes)
    want_s = np.zeros_like(scales)
    for (s, r), t in rows.items():
        want_c[s, r] = gc[s, t]
        want_s[s, r] = gs[s, t]
    np.testing.assert_array_equal(codes, want_c)
    np.testing.assert_array_equal(scales, want_s)
    assert len(rows) == 3 * 9 * 3 - 2


# ---------------------------------------------------------------------------
# Combine with partial sums on the expert side ("Evaluation": the sender-side
# accumulation that receiver-only accumulation is contrasted with)
# ---------------------------------------------------------------------------

def _one(v: int) -> np.ndarray:
    return np.array([v], np.uint16)


BF16_ONE, BF16_2M8, BF16_2M25 = 0x3F80, 0x3B80, 0x3300      # 1, 2^-8, 2^-25


def test_presum_groups_by_rank_and_rounds_each_partial():
    """Weights 1; slot 0 (2^-8) on rank 0, slots 1 (1) and 2 (2^-8) on rank 1.
    Rank 1's partial 1 + 2^-8 is a bf16 tie and rounds to 1; the final
    2^-8 + 1 is a tie again: 1 (0x3F80). Receiver-only accumulation gives
    1 + 2^-7 (0x3F81), and so do three separate ranks (exact partials)."""
    w = np.ones(3, np.float32)
    rows = [_one(BF16_2M8), _one(BF16_ONE), _one(BF16_2M8)]
    assert oracle.combine_presum_token(w, rows, [0, 1, 1])[0] == 0x3F80
    assert oracle.combine_token(w, rows)[0] == 0x3F81
    assert oracle.combine_presum_token(w, rows, [0, 1, 2])[0] == 0x3F81
    assert oracle.combine_presum_token(np.array([0.25, 0.75], np.float32),
                                       [None, _one(BF16_ONE)], [None, 0])[0] == 0x3F40


def test_presum_adds_partials_in_slot_order():
    """Partials 1, 2^-8, 2^-25 x 3 on five ranks. Added from slot 0 upward,
    each 2^-25 is a quarter ulp of 1 + 2^-8 in float and is lost, leaving a
    bf16 tie that rounds to 1. In the opposite order the small ones add up
    to 3 * 2^-25 first and the float sum 1 + 2^-8 + 2^-23 rounds to 1 + 2^-7.
    The ranks run 4..0, so rank order would be the opposite order."""
    w = np.ones(5, np.float32)
    rows = [_one(BF16_ONE), _one(BF16_2M8)] + [_one(BF16_2M25)] * 3
    assert oracle.combine_presum_token(w, rows, [4, 3, 2, 1, 0])[0] == 0x3F80
    assert oracle.combine_presum_token(w, rows[::-1], [0, 1, 2, 3, 4])[0] == 0x3F81


def test_presum_single_choice_is_the_rounded_product():
    """R = 1: every group is one slot, the partial is bf16(float(w * y)) (a
    correctly rounded float product, here from numpy, then torch's bf16
    cast), and the final sum returns it unchanged; the partial sits in the
    token's only slot row."""
    sh = W.Shape("r1", 4, 16, 64, 8, 1, expert="scale", seed=3)
    wl = W.make_workload(sh)
    r = oracle.run(wl)
    p = r["plan"]
    partial, out = oracle.combine_presum(r["y"], wl.weights, wl.idx, p)
    L = sh.n_experts // sh.n_ranks
    y = r["y"][wl.idx[..., 0] // L, p["grp_pos"][..., 0]]          # [N, T, H]
    prod = wl.weights[..., 0:1].astype(np.float32) * W.bf16_bits_to_f32(y)
    want = W.to_bf16_bits(prod.astype(np.float32))
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(partial, out)


def test_presum_one_rank_exact_sums_equal_the_plain_combine():
    """N = 1: all of a token's slots form one group. With power-of-two
    weights and values of magnitude in [2^-4, 2) every product and float sum
    is exact, so the result is the correctly rounded exact sum: the plain
    combine's value (double accumulation, one rounding)."""
    sh = W.Shape("one_rank", 1, 64, 96, 6, 4, seed=5)
    wl = W.make_workload(sh)
    rng = np.random.default_rng(5)
    mag = rng.uniform(2.0 ** -4, 2.0, size=wl.x_bf16.shape)
    sign = rng.choice([-1.0, 1.0], size=wl.x_bf16.shape)
    wl.x_bf16 = W.to_bf16_bits((mag * sign).astype(np.float32))
    wl.planes = [wl.x_bf16.view(np.uint8).reshape(1, 64, 2 * 96)]
    wl.weights = rng.choice([0.5, 0.25, 0.125, 0.0625], size=wl.weights.shape).astype(np.float32)
    r = oracle.run(wl)
    partial, out = oracle.combine_presum(r["y"], wl.weights, wl.idx, r["plan"])
    np.testing.assert_array_equal(out, r["out"])
    np.testing.assert_array_equal(partial[0, ::4], out[0])        # leader = slot 0


def test_presum_partial_rows_sit_at_group_leaders():
    """Hand layout: N = 2, E = 4 (experts 0, 1 on rank 0; 2, 3 on rank 1),
    one token of rank 0 routed to experts (0, 2, 3) with weights 1 and expert
    rows 2^-8, 1, 2^-8: rank 1 holds slots 1 and 2 (different experts), so
    its partial (1 + 2^-8 rounded to 1) sits in slot 1's row, slot 2's row is
    left untouched, and the token combines to 1 (0x3F80)."""
    N, T, E, R, H = 2, 1, 4, 3, 1
    idx = np.array([[[0, 2, 3]], [[1, 0, 1]]], np.int32)
    p = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), idx)
    cap = oracle.recv_bound(N, T, E, R)
    y = np.zeros((N, cap, H), np.uint16)
    vals = [BF16_2M8, BF16_ONE, BF16_2M8]
    for k in range(R):
        y[idx[0, 0, k] // 2, p["grp_pos"][0, 0, k], 0] = vals[k]
    w = np.ones((N, T, R), np.float32)
    partial, out = oracle.combine_presum(y, w, idx, p)
    assert out[0, 0, 0] == 0x3F80
    assert list(partial[0, :, 0]) == [BF16_2M8, BF16_ONE, 0]


# ---------------------------------------------------------------------------
# KV-block push: regions and the copy
# ---------------------------------------------------------------------------

def _read_kv_golden():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_regions.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    n, tok, bs_src, bs_dst = map(int, rows[0])
    src = np.array(rows[1], np.int32)
    dst = np.array(rows[2], np.int32)
    regions = np.array([list(map(int, r)) for r in rows[3:]], np.int64)
    return n, tok, bs_src, src, bs_dst, dst, regions


def test_kv_regions_hand_worked_example():
    n, tok, bs_src, src, bs_dst, dst, want = _read_kv_golden()
    np.testing.assert_array_equal(oracle.kv_regions(n, tok, bs_src, src, bs_dst, dst), want)


def _block_runs(src, dst):
    """Maximal runs of block indices where both tables step by one."""
    breaks = (np.diff(src) != 1) | (np.diff(dst) != 1)
    return 1 + int(breaks.sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kv_regions_equal_block_sizes_count_block_runs(seed):
    """Same block size on both sides: a region can only break at a block
    boundary, and does exactly where either table stops stepping by one."""
    rng = np.random.default_rng(seed)
    bs, tok = 4, 32
    nb = 50
    src = rng.permutation(200)[:nb].astype(np.int32)
    src[10:20] = np.arange(70, 80)                     # a long adjacent stretch
    dst = rng.permutation(300)[:nb].astype(np.int32)
    dst[10:20] = np.arange(7, 17)
    n = nb * bs - 3                                    # last block partly used
    reg = oracle.kv_regions(n, tok, bs, src, bs, dst)
    assert reg.shape[0] == _block_runs(src, dst)
    assert reg[:, 2].sum() == n * tok


def test_kv_regions_identity_tables_are_one_region():
    n, tok = 1000, 48
    reg = oracle.kv_regions(n, tok, 16, np.arange(63, dtype=np.int32), 1,
                            np.arange(1000, dtype=np.int32))
    np.testing.assert_array_equal(reg, [[0, 0, n * tok]])


@pytest.mark.parametrize("bs_src,bs_dst", [(1, 1), (4, 16), (16, 4), (3, 5)])
def test_kv_copy_puts_each_token_where_the_tables_say(bs_src, bs_dst):
    """Pools as arrays [blocks, block_tokens, token_bytes]: after the copy,
    destination token i (block dst[i / bs], slot i % bs) holds source token
    i's bytes, on every rank; nothing else changes. Regions tile the tokens
    in order and no two neighbours could be merged."""
    rng = np.random.default_rng(bs_src * 31 + bs_dst)
    ranks, tok, n = 3, 16, 97
    nsb, ndb = 200 // bs_src + 40, 200 // bs_dst + 40
    sblocks = rng.permutation(nsb)[: -(-n // bs_src)].astype(np.int32)
    dblocks = rng.permutation(ndb)[: -(-n // bs_dst)].astype(np.int32)
    sblocks[2:6] = np.arange(4) + nsb - 8 if len(sblocks) > 6 else sblocks[2:6]
    src = rng.integers(0, 256, size=(ranks, nsb * bs_src * tok), dtype=np.uint8)
    dst = rng.integers(0, 256, size=(ranks, ndb * bs_dst * tok), dtype=np.uint8)
    reg = oracle.kv_regions(n, tok, bs_src, sblocks, bs_dst, dblocks)
    got = oracle.kv_copy(reg, src, dst)
    sv = src.reshape(ranks, nsb, bs_src, tok)
    want = dst.copy().reshape(ranks, ndb, bs_dst, tok)
    for i in range(n):
        want[:, dblocks[i // bs_dst], i % bs_dst] = sv[:, sblocks[i // bs_src], i % bs_src]
    np.testing.assert_array_equal(got, want.reshape(ranks, -1))
    assert reg[:, 2].sum() == n * tok
    ends = reg[:-1, :2] + reg[:-1, 2:3]
    assert not ((ends[:, 0] == reg[1:, 0]) & (ends[:, 1] == reg[1:, 1])).any()

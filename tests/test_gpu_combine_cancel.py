"""ep_combine on expert rows whose terms cancel, against the oracle, every
element.

The workloads' stand-in experts (identity, scale, dequantise) give a token R
terms of one sign. A grouped GEMM's outputs ("Enabling trillion-parameter
models on AWS EFA", section "Dispatch and combine": combine takes the expert
outputs back to their tokens) have mixed signs, so here the expert output
buffer is filled with random mixed-sign bf16 rows instead. Bar: the
cancellation-aware combine_close (8e-3 relative plus an absolute term from
fp32 accumulation), on every output element, for both shapes of the combine
kernel (two waves per token below 16384 tokens, seven at and above).
"""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import (abs_term_sum, combine_close, desc_of, note, plan_arrays, random_bf16,
                      upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _plan_on_gpu(sh, wl):
    """ep_plan with the capacity set to the largest delivered count (so the
    expert output buffer holds no unused rows); its tables equal the
    oracle's."""
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    full = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), wl.idx)
    cap = max(1, int(full["recv_off"][:, N].max()))
    d = desc_of(sh, cap)
    p = oracle.plan(N, T, E, R, cap, wl.idx)
    b = ep.Buffers(d)
    upload(b, wl)
    b.status.zero_()
    ep.plan(d, b.idx, b.plan_ws, b.status)
    torch.cuda.synchronize()
    got = plan_arrays(d, b)
    for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    return d, b, p, cap


def _check_combine(d, b, p, y, weights, idx, L):
    """Run ep_combine on expert rows y (bf16 bits [N, cap, H], host) and
    compare every element with the oracle's combine."""
    b.expert_out.copy_(torch.from_numpy(y.view(np.int16)))
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    torch.cuda.synchronize()
    want = oracle.combine(y, weights, idx, p)
    got = b.out.cpu().numpy().view(np.uint16)
    N, T, R = idx.shape
    gp = p["grp_pos"]
    bad_total = 0
    for s in range(N):
        ok_slot = (idx[s] >= 0) & (gp[s] >= 0)
        owner = np.where(ok_slot, idx[s] // L, 0)
        ys = y[owner, np.where(ok_slot, gp[s], 0)]               # [T, R, H]
        ys[~ok_slot] = 0
        S = abs_term_sum(weights[s], ys)
        ok = combine_close(got[s], want[s], S, R)
        bad_total += int((~ok).sum())
    assert bad_total == 0, f"{bad_total} elements outside the bar"
    return got, want


def _random_expert_rows(rng, p, cap, H, N):
    y = np.zeros((N, cap, H), np.uint16)
    for dd in range(N):
        n = min(int(p["recv_off"][dd, N]), cap)
        y[dd, :n] = random_bf16(rng, (n, H))
    return y


def test_combine_mixed_sign_decode_shape():
    """Decode shape (32 x 128 tokens, H 7168, top-8 of 256): random rows, and
    in every other token the last slot's row set to cancel the first seven
    (y_7 = bf16(-sum_{k<7} w_k y_k / w_7))."""
    sh = W.Shape("cancel_decode", 32, 128, 7168, 256, 8, seed=31)
    wl = W.make_workload(sh)
    N, T, H, R, L = 32, 128, 7168, 8, 8
    note("combine cancellation, decode shape")
    d, b, p, cap = _plan_on_gpu(sh, wl)
    rng = np.random.default_rng(32)
    y = _random_expert_rows(rng, p, cap, H, N)
    own = wl.idx // L
    gp = p["grp_pos"]
    for s in range(N):
        for t in range(0, T, 2):
            head = np.zeros(H, np.float64)
            for k in range(R - 1):
                head += float(wl.weights[s, t, k]) * W.bf16_bits_to_f32(
                    y[own[s, t, k], gp[s, t, k]]).astype(np.float64)
            last = (-head / float(wl.weights[s, t, R - 1])).astype(np.float32)
            y[own[s, t, R - 1], gp[s, t, R - 1]] = W.to_bf16_bits(last)
    got, want = _check_combine(d, b, p, y, wl.weights, wl.idx, L)
    assert (want == 0).sum() + (np.abs(W.bf16_bits_to_f32(want)) < 1e-3).sum() > 0


def test_combine_mixed_sign_many_tokens():
    """16384 tokens (the seven-waves-per-token kernel), H 7168, top-4 of 16,
    with 1% of the slots dropped (bad ids)."""
    sh = W.Shape("cancel_many", 4, 4096, 7168, 16, 4, seed=33)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    rng = np.random.default_rng(34)
    idx[rng.random(idx.shape) < 0.01] = -1
    wl = W.make_workload(sh, idx=idx)
    note("combine cancellation, 16384 tokens")
    d, b, p, cap = _plan_on_gpu(sh, wl)
    assert p["status"] == oracle.STATUS_BAD_EXPERT
    y = _random_expert_rows(rng, p, cap, 7168, 4)
    _check_combine(d, b, p, y, wl.weights, wl.idx, 4)


def test_combine_exact_pair_cancellation():
    """Equal weights in pairs and opposite rows: every exact sum is 0 (the
    oracle's +0); the GPU keeps at most a product's fp32 rounding error."""
    sh = W.Shape("cancel_pairs", 4, 64, 1024, 16, 4, seed=35)
    wl = W.make_workload(sh)
    w = np.repeat(np.random.default_rng(36).dirichlet(np.ones(2), size=(4, 64)) / 2, 2,
                  axis=-1).astype(np.float32)
    wl.weights = w
    note("combine exact pair cancellation")
    d, b, p, cap = _plan_on_gpu(sh, wl)
    rng = np.random.default_rng(37)
    y = _random_expert_rows(rng, p, cap, 1024, 4)
    own, gp = wl.idx // 4, p["grp_pos"]
    for k in (1, 3):
        y[own[..., k], gp[..., k]] = y[own[..., k - 1], gp[..., k - 1]] ^ np.uint16(0x8000)
    got, want = _check_combine(d, b, p, y, w, wl.idx, 4)
    assert (want == 0).all()

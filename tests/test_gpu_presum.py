"""Combine with partial sums on the expert side, against the CPU oracle.

Both sides take the same IEEE operations in the same order (fp32 fused
multiply-adds in slot order per group, one bf16 rounding per group, fp32
adds of the partials in leader order, one final rounding), so partial rows
and outputs must match bit for bit. At full size, sampled tokens are
checked against the oracle, and every sampled element against the error
bound of the two-level rounding relative to the exact weighted sum.
"""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import desc_of, note, plan_arrays, rows_of, run_path, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _presum(d, b):
    N, T, R, H = d.n_ranks, d.tokens, d.topk, d.hidden
    partial = torch.zeros((N, T * R, H), dtype=torch.int16, device="cuda")
    out = torch.full((N, T, H), 0x7FC0, dtype=torch.int16, device="cuda")
    ep.combine_presum(d, b.expert_out, b.weights, b.plan_ws, partial, out)
    torch.cuda.synchronize()
    return partial, out


PRESUM_SHAPES = [
    W.CONFIGS["tiny"], W.CONFIGS["tiny_zipf"],
    W.Shape("single_rank", 1, 37, 64, 5, 2),
    W.Shape("topk1", 4, 50, 128, 8, 1),
    W.Shape("rank0_repeated_ids", 8, 8, 64, 32, 8, routing="rank0"),
    W.Shape("few_ranks_many_choices", 2, 40, 512, 16, 6, expert="scale", seed=8),
    W.Shape("max_experts", 2, 64, 64, 2048, 16),
    W.Shape("max_topk", 2, 8, 64, 128, 64, expert="scale", seed=3),
    W.Shape("many_ranks", 128, 4, 64, 128, 4, routing="zipf"),
    W.Shape("zipf_mid", 16, 64, 512, 128, 6, routing="zipf", expert="scale"),
    W.Shape("fp8_h1024", 4, 12, 1024, 16, 4, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("wide_row", 2, 5, 8192, 4, 2, expert="scale"),
    W.Shape("no_tokens", 2, 0, 64, 4, 2),
]


def check_presum(sh, wl, cap=0):
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    note(f"presum {sh.name} N={sh.n_ranks} T={sh.tokens} H={sh.hidden} E={sh.n_experts} "
         f"R={sh.topk} cap={cap}")
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    partial, out = _presum(d, b)
    ref = oracle.run(wl, cap=cap)
    assert int(b.status.item()) == ref["plan"]["status"]
    want_partial, want_out = oracle.combine_presum(ref["y"], wl.weights, wl.idx, ref["plan"])
    np.testing.assert_array_equal(partial.cpu().numpy().view(np.uint16), want_partial)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want_out)
    return d, b, out


@pytest.mark.parametrize("sh", PRESUM_SHAPES, ids=[s.name for s in PRESUM_SHAPES])
def test_presum_full(sh):
    check_presum(sh, W.make_workload(sh))


def test_presum_dropped_slots():
    sh = W.Shape("bad_tight", 4, 32, 128, 16, 3, routing="zipf", expert="scale", seed=12)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    idx[0, 0, 0] = 16
    idx[2, 7, :] = -1                      # a token with no delivered slot: zeros
    wl = W.make_workload(sh, idx=idx)
    full = oracle.plan(4, 32, 16, 3, oracle.recv_bound(4, 32, 16, 3), wl.idx)
    cap = int(full["recv_off"][:, 4].max()) - 5
    d, b, out = check_presum(sh, wl, cap=cap)
    assert int(b.status.item()) == ep.EP_STATUS_BAD_EXPERT | ep.EP_STATUS_CAPACITY
    assert not out[2, 7].any()


def test_presum_single_choice_equals_plain_combine():
    """R = 1: one slot per group, so both combines compute bf16(float(w * y))."""
    sh = W.Shape("r1", 8, 64, 512, 32, 1, expert="scale", seed=2)
    wl = W.make_workload(sh)
    d = desc_of(sh)
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    _, out = _presum(d, b)
    assert torch.equal(out, b.out)


@pytest.mark.parametrize("name", ["decode", "prefill", "worst"])
def test_presum_full_size(name):
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    d = desc_of(sh)
    N, T, R, H, E = sh.n_ranks, sh.tokens, sh.topk, sh.hidden, sh.n_experts
    L = E // N
    note(f"presum full-size {name}")
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    partial, out = _presum(d, b)
    assert int(b.status.item()) == 0
    p = plan_arrays(d, b)
    rng = np.random.default_rng(4)
    toks = rng.choice(N * T, size=48, replace=False)
    s, t = np.unravel_index(toks, (N, T))
    got = rows_of(out, s, t).view(np.uint16)
    cap = ep.capacity(d)
    worst = 0.0
    for i in range(len(toks)):
        e = wl.idx[s[i], t[i]]
        g = p["comb_row"][s[i], t[i]]
        ys = rows_of(b.expert_out, (g // cap).astype(np.int64), (g % cap).astype(np.int64))
        ys = [y.view(np.uint16) for y in ys]
        want = oracle.combine_presum_token(wl.weights[s[i], t[i]], ys, list(e // L))
        np.testing.assert_array_equal(got[i], want, err_msg=f"token {s[i]},{t[i]}")
        # error bound against the exact weighted sum: one bf16 rounding per
        # partial and one at the end (unit roundoff 2^-8 each), plus fp32 slack
        yf = np.stack([W.bf16_bits_to_f32(y).astype(np.float64) for y in ys])
        wk = wl.weights[s[i], t[i]].astype(np.float64)[:, None]
        exact = (wk * yf).sum(0)
        mag = np.abs(wk * yf).sum(0)
        err = np.abs(W.bf16_bits_to_f32(got[i]).astype(np.float64) - exact)
        bound = 2.0 ** -8 * np.abs(exact) + (2.0 ** -8 + 2.0 ** -20) * mag
        assert (err <= bound).all(), f"token {s[i]},{t[i]}"
        worst = max(worst, float((err / np.maximum(mag, 1e-30)).max()))
    note(f"presum {name}: max |err| / sum |w y| over sampled tokens = {worst:.3e}")

"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bar: plan tables and every moved byte bit-exact; combine within 8e-3
relative per element (fp32 accumulation on the GPU against the oracle's
single rounding of the exact sum; one bf16 ulp is at most 2^-7 relative).
Small workloads are compared element by element in full; the full-size
workloads compare every plan table in full, sampled rows and tokens that the
oracle computes one by one, and whole-tensor properties (closed forms).
"""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import (bf16_close, desc_of, expected_plan_extras, expected_win_list, note,
                      plan_arrays, rows_of, run_path, tok_bytes_of, upload)

pytestmark = pytest.mark.gpu

ORACLE_PLAN = ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos")


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _identity_exact(sh, wl):
    return (sh.expert == "identity" and bool((wl.idx >= 0).all())
            and bool((wl.idx < sh.n_experts).all()))


def compare_full(sh, wl, cap=0, staged=False, check_closed_form=True):
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    N, T, E, R, H = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk, sh.hidden
    note(f"full parity {sh.name} N={N} T={T} H={H} E={E} R={R} cap={cap} staged={staged}")
    b = ep.Buffers(d, staged=staged)
    upload(b, wl)
    run_path(d, b, wl, staged=staged)
    torch.cuda.synchronize()
    ref = oracle.run(wl, cap=cap)
    p = ref["plan"]
    assert int(b.status.item()) == p["status"]
    got = plan_arrays(d, b)
    for f in ORACLE_PLAN:
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    for f, v in expected_plan_extras(p, wl.idx, N, E, cap).items():
        np.testing.assert_array_equal(got[f], v, err_msg=f)
    wlist = expected_win_list(p, N, T, R, tok_bytes_of(d))
    assert (wlist is None) == ("win_list" not in got)
    if wlist is not None:
        np.testing.assert_array_equal(got["win_list"], wlist, err_msg="win_list")
    totals = p["recv_off"][:, N]
    for q in range(len(wl.planes)):
        send = b.send[q].cpu().numpy()
        for s in range(N):
            n = p["send_off"][s, E]
            np.testing.assert_array_equal(send[s, :n], ref["send"][q][s, :n], err_msg=f"send {s}")
        grouped = b.grouped[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(grouped[dd, :n], ref["grouped"][q][dd, :n],
                                          err_msg=f"grouped {dd}")
        if staged:
            recv = b.recv[q].cpu().numpy()
            for dd in range(N):
                n = min(int(totals[dd]), cap)
                np.testing.assert_array_equal(recv[dd, :n], ref["recv"][q][dd, :n],
                                              err_msg=f"recv {dd}")
    y = b.expert_out.cpu().numpy().view(np.uint16)
    for dd in range(N):
        n = min(int(totals[dd]), cap)
        np.testing.assert_array_equal(y[dd, :n], ref["y"][dd, :n], err_msg=f"expert {dd}")
    out = b.out.cpu().numpy().view(np.uint16)
    ok = bf16_close(out, ref["out"])
    assert ok.all(), f"combine: {int((~ok).sum())} elements off, first {np.argwhere(~ok)[:3]}"
    if check_closed_form and _identity_exact(sh, wl) and p["status"] == 0:
        # identity experts: out == x as numbers (+0 for -0 inputs)
        np.testing.assert_array_equal(_unsign_zero(out), _unsign_zero(wl.x_bf16))
    return d, b, ref


@pytest.mark.parametrize("name", ["tiny", "tiny_zipf"])
@pytest.mark.parametrize("staged", [False, True])
def test_small_configs_full(name, staged):
    sh = W.CONFIGS[name]
    compare_full(sh, W.make_workload(sh), staged=staged)


EDGE_SHAPES = [
    W.Shape("single_rank", 1, 37, 64, 5, 2),
    W.Shape("topk1", 4, 50, 128, 8, 1),
    W.Shape("one_expert_per_rank", 8, 20, 136, 8, 3),
    W.Shape("mostly_empty_experts", 4, 8, 64, 64, 2),
    W.Shape("rank0_repeated_ids", 8, 8, 64, 32, 8, routing="rank0"),
    W.Shape("multi_chunk_plan", 2, 3000, 64, 12, 3, expert="scale"),
    W.Shape("wide_row_two_passes", 2, 5, 8192, 4, 2),
    W.Shape("ragged_row", 3, 7, 1000, 6, 2, expert="scale"),
    W.Shape("no_tokens", 2, 0, 64, 4, 2),
    W.Shape("fp8_dword_scales", 2, 9, 256, 8, 2, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("fp8_h1024", 4, 12, 1024, 16, 4, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("max_experts", 2, 64, 64, 2048, 16),
    W.Shape("max_topk", 2, 8, 64, 128, 64, expert="scale", seed=3),   # EP_MAX_TOPK
    W.Shape("many_ranks", 128, 4, 64, 128, 4, routing="zipf"),
    W.Shape("zipf_mid", 16, 64, 512, 128, 6, routing="zipf", expert="scale"),
    # 16800 tokens: the combine's many-token shape (7 waves per token), with
    # ragged 400-byte rows and a multi-chunk plan, compared in full
    W.Shape("many_tokens_ragged", 4, 4200, 200, 16, 3, expert="scale", seed=6),
    # Sources of 4 to 32 MiB of token rows take the windowed sender (the last
    # window partial for 600 and 300 tokens), larger ones the token-order
    # sender: one pass of 14 chunks per lane, the two-plane fp8 form, and
    # the general kernel (rows over 14 KB).
    W.Shape("large_source_bf16", 2, 512, 4608, 16, 8, expert="scale"),
    W.Shape("large_source_fp8", 2, 600, 7168, 16, 8, payload=W.PAYLOAD_FP8_B128,
            expert="dequant"),
    W.Shape("large_source_wide_row", 2, 300, 8192, 4, 2),
    # windowed with 2048 experts (the list kernel scans more entries than it
    # has threads) and with skewed routing (experts empty inside a window)
    W.Shape("large_source_max_experts", 2, 600, 4608, 2048, 8),
    W.Shape("large_source_zipf", 4, 400, 7168, 64, 6, routing="zipf", expert="scale", seed=9),
    W.Shape("huge_source_bf16", 2, 4200, 4096, 16, 4, expert="scale"),
    W.Shape("huge_source_fp8", 2, 4600, 7168, 16, 4, payload=W.PAYLOAD_FP8_B128,
            expert="dequant"),
    W.Shape("huge_source_wide_row", 2, 2100, 8192, 4, 2),
]


@pytest.mark.parametrize("sh", EDGE_SHAPES, ids=[s.name for s in EDGE_SHAPES])
def test_edge_shapes_full(sh):
    compare_full(sh, W.make_workload(sh))


@pytest.mark.parametrize("sh", EDGE_SHAPES[:6], ids=[s.name for s in EDGE_SHAPES[:6]])
def test_edge_shapes_staged(sh):
    compare_full(sh, W.make_workload(sh), staged=True)


def _bad_and_tight():
    sh = W.Shape("bad_ids", 4, 32, 128, 16, 3, expert="scale", seed=11)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    idx[0, 0, 0] = 16
    idx[1, 5, 2] = -3
    idx[3, 31, 1] = 1 << 20
    return sh, W.make_workload(sh, idx=idx)


def test_windowed_sender_with_bad_ids_and_tight_capacity():
    """Dropped slots leave gaps in a window's list; a tight capacity drops
    rows on the receive side only."""
    sh = W.Shape("window_bad", 2, 600, 4608, 16, 8, expert="scale", seed=5)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    rng = np.random.default_rng(7)
    bad = rng.random(idx.shape) < 0.02
    idx[bad] = rng.choice([-1, 16, 99], size=int(bad.sum()))
    wl = W.make_workload(sh, idx=idx)
    full = oracle.plan(2, 600, 16, 8, oracle.recv_bound(2, 600, 16, 8), idx)
    cap = int(full["recv_off"][:, 2].max()) - 3
    compare_full(sh, wl, cap=cap)


def test_bad_expert_ids_are_dropped_and_flagged():
    sh, wl = _bad_and_tight()
    d, b, ref = compare_full(sh, wl)
    assert int(b.status.item()) == ep.EP_STATUS_BAD_EXPERT


def test_capacity_overflow_drops_rows_and_flags():
    sh = W.Shape("tight", 4, 32, 128, 16, 3, routing="zipf", expert="scale", seed=12)
    wl = W.make_workload(sh)
    full = oracle.plan(4, 32, 16, 3, oracle.recv_bound(4, 32, 16, 3), wl.idx)
    cap = int(full["recv_off"][:, 4].max()) - 5          # the busiest rank overflows
    d, b, ref = compare_full(sh, wl, cap=cap)
    assert int(b.status.item()) & ep.EP_STATUS_CAPACITY
    assert (ref["plan"]["grp_pos"] == -1).sum() >= 5


def _staged_overflow_idx(N, T, L):
    """Routing whose rows lost by rank 0's receive buffer sit early in its
    grouped order: sources 0 .. N-2 send every token to rank 0's expert 1,
    the last source to its expert 0 (second choices go to other ranks)."""
    idx = np.zeros((N, T, 2), np.int32)
    idx[:, :, 0] = 1
    idx[N - 1, :, 0] = 0
    idx[:, :, 1] = L + (np.arange(N)[:, None] % (N - 1)) * L + np.arange(T)[None, :] % L
    return idx


STAGED_OVERFLOW = [
    (W.Shape("tight_staged", 4, 32, 128, 16, 3, routing="zipf", expert="scale", seed=13), None),
    (W.Shape("tight_staged_early", 4, 24, 256, 16, 2, expert="scale", seed=15), "early"),
    (W.Shape("tight_staged_fp8", 4, 24, 256, 16, 2, payload=W.PAYLOAD_FP8_B128,
             expert="dequant", seed=16), "early"),
]


@pytest.mark.parametrize("sh,routing", STAGED_OVERFLOW, ids=[c[0].name for c in STAGED_OVERFLOW])
def test_capacity_overflow_staged_path(sh, routing):
    """Staged path under overflow: the receive buffer keeps the first cap
    rows of each rank in receive order and the unpack writes zeros into the
    grouped rows whose receive row was lost. Receive buffers, grouped
    layouts, expert outputs and the combine, compared in full with the
    oracle's transfer into a cap-row receive buffer, its unpack, expert and
    combine."""
    N, T, E, R, H = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk, sh.hidden
    wl = W.make_workload(sh)
    if routing == "early":
        wl = W.make_workload(sh, idx=_staged_overflow_idx(N, T, E // N))
    full = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), wl.idx)
    cap = int(full["recv_off"][:, N].max()) - 4
    d = desc_of(sh, cap)
    note(f"staged overflow {sh.name} cap={cap}")
    b = ep.Buffers(d, staged=True)
    upload(b, wl)
    for g in b.grouped:
        g.fill_(0x5A)                             # stale bytes must not survive
    run_path(d, b, wl, staged=True)
    torch.cuda.synchronize()
    p = oracle.plan(N, T, E, R, cap, wl.idx)
    assert int(b.status.item()) == p["status"] and p["status"] & ep.EP_STATUS_CAPACITY
    send = [oracle.dispatch_pack(pl, p) for pl in wl.planes]
    recv = [oracle.transfer(sp, p, cap) for sp in send]
    grouped = [oracle.unpack(r, p, cap) for r in recv]
    y = oracle.expert_op(grouped, p, H, sh.payload, wl.alpha)
    out = oracle.combine(y, wl.weights, wl.idx, p)
    zero_rows = 0
    for q in range(len(wl.planes)):
        r_got = b.recv[q].cpu().numpy()
        g_got = b.grouped[q].cpu().numpy()
        for dd in range(N):
            n = min(int(p["recv_off"][dd, N]), cap)
            np.testing.assert_array_equal(r_got[dd, :n], recv[q][dd, :n], err_msg=f"recv {dd}")
            np.testing.assert_array_equal(g_got[dd, :n], grouped[q][dd, :n],
                                          err_msg=f"grouped {dd}")
            if q == 0:
                zero_rows += int((grouped[0][dd, :n] == 0).all(axis=1).sum())
    if routing == "early":
        assert zero_rows >= 4                     # lost receive rows below cap
    y_got = b.expert_out.cpu().numpy().view(np.uint16)
    for dd in range(N):
        n = min(int(p["recv_off"][dd, N]), cap)
        np.testing.assert_array_equal(y_got[dd, :n], y[dd, :n], err_msg=f"expert {dd}")
    ok = bf16_close(b.out.cpu().numpy().view(np.uint16), out)
    assert ok.all(), f"combine: {int((~ok).sum())} elements off"


def test_deterministic_and_stream_independent():
    sh = W.CONFIGS["decode_zipf"]
    sh = W.Shape("det", 16, 96, 1024, 128, 8, routing="zipf", expert="scale", seed=5)
    wl = W.make_workload(sh)
    d = desc_of(sh)
    note("determinism: two runs, second on a side stream")
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    torch.cuda.synchronize()
    first = [b.plan_ws.clone(), b.send[0].clone(), b.out.clone()]
    grouped_first = b.grouped[0].clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b.send[0].zero_()
        b.out.zero_()
        run_path(d, b, wl, stream=s)
    s.synchronize()
    # the chunk-count scratch is recomputed, so the whole workspace repeats
    assert torch.equal(first[0], b.plan_ws)
    assert torch.equal(first[1], b.send[0])
    assert torch.equal(first[2], b.out)
    assert torch.equal(grouped_first, b.grouped[0])


def test_host_pointer_is_rejected():
    sh = W.CONFIGS["tiny"]
    d = desc_of(sh)
    b = ep.Buffers(d)
    host_idx = torch.zeros((4, 16, 2), dtype=torch.int32)
    with pytest.raises(ep.EPError) as e:
        ep.plan(d, host_idx, b.plan_ws, b.status)
    assert e.value.code == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EPError):
        ep.dispatch_pack(d, [b.x[0], b.x[0]], b.plan_ws, b.send)   # plane 1 must be NULL


def test_probe_copy():
    src = torch.randint(0, 255, (3 * 14336 * 97 + 48,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    ep.probe_copy(dst, src, src.numel())
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ---------------------------------------------------------------------------
# Full-size workloads (the configurations of the benchmark and its siblings)
# ---------------------------------------------------------------------------

def compare_full_size(name, n_slots=3000, n_tokens=300, full_oracle=False):
    """Plan tables in full, every send and delivered grouped row on the
    device, sampled rows and tokens against the oracle one by one; with
    full_oracle also the oracle's whole path (plan, pack, transfer, unpack,
    expert, combine): every expert-output row and every output token."""
    sh = W.CONFIGS[name]
    N, T, E, R, H = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk, sh.hidden
    L = E // N
    wl = W.make_workload(sh)
    d = desc_of(sh)
    cap = ep.capacity(d)
    note(f"full-size {name} N={N} T={T} H={H} E={E} R={R} cap={cap}")
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    torch.cuda.synchronize()
    p = oracle.plan(N, T, E, R, cap, wl.idx)
    assert int(b.status.item()) == p["status"] == 0
    got = plan_arrays(d, b)
    for f in ORACLE_PLAN:
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    for f, v in expected_plan_extras(p, wl.idx, N, E, cap).items():
        np.testing.assert_array_equal(got[f], v, err_msg=f)
    # every send row and every delivered grouped row, on the device, against
    # the token row the oracle's plan puts there
    ss, tt_, kk = np.unravel_index(np.arange(N * T * R), (N, T, R))
    ee = wl.idx.reshape(-1)
    for q in range(len(wl.planes)):
        for lo in range(0, N * T * R, 8192):
            sl = slice(lo, min(lo + 8192, N * T * R))
            si = torch.from_numpy(ss[sl]).cuda()
            ti = torch.from_numpy(tt_[sl]).cuda()
            want = b.x[q][si, ti]
            spi = torch.from_numpy(p["send_pos"].reshape(-1)[sl].astype(np.int64)).cuda()
            gpi = torch.from_numpy(p["grp_pos"].reshape(-1)[sl].astype(np.int64)).cuda()
            di = torch.from_numpy((ee[sl] // L).astype(np.int64)).cuda()
            assert torch.equal(b.send[q][si, spi], want), f"send rows {lo}.."
            assert torch.equal(b.grouped[q][di, gpi], want), f"grouped rows {lo}.."
    rng = np.random.default_rng(123)
    slots = rng.choice(N * T * R, size=min(N * T * R, n_slots), replace=False)
    s, t, k = np.unravel_index(slots, (N, T, R))
    e = wl.idx[s, t, k]
    dst = e // L
    gp = p["grp_pos"][s, t, k]
    sp = p["send_pos"][s, t, k]
    for q, plane in enumerate(wl.planes):
        want = plane[s, t]
        np.testing.assert_array_equal(rows_of(b.send[q], s, sp), want, err_msg=f"send plane {q}")
        np.testing.assert_array_equal(rows_of(b.grouped[q], dst, gp), want,
                                      err_msg=f"grouped plane {q}")
    y = rows_of(b.expert_out, dst, gp).view(np.uint16)
    for i in range(len(slots)):
        row = [pl[s[i], t[i]] for pl in wl.planes]
        np.testing.assert_array_equal(y[i], oracle.expert_row(row, int(e[i]), sh.payload, H, wl.alpha))
    toks = rng.choice(N * T, size=min(N * T, n_tokens), replace=False)
    ts, tt = np.unravel_index(toks, (N, T))
    out = rows_of(b.out, ts, tt).view(np.uint16)
    for i in range(len(toks)):
        row = [pl[ts[i], tt[i]] for pl in wl.planes]
        ys = [oracle.expert_row(row, int(ee), sh.payload, H, wl.alpha) for ee in wl.idx[ts[i], tt[i]]]
        want = oracle.combine_token(wl.weights[ts[i], tt[i]], ys)
        assert bf16_close(out[i], want).all(), (name, ts[i], tt[i])
    if full_oracle:
        ref = oracle.run(wl, cap=cap)
        rows = ref["rows"]
        y_got = b.expert_out[:, :rows].cpu().numpy().view(np.uint16)
        for dd in range(N):
            n = min(int(p["recv_off"][dd, N]), cap)
            np.testing.assert_array_equal(y_got[dd, :n], ref["y"][dd, :n], err_msg=f"expert {dd}")
        del y_got
        ok = bf16_close(b.out.cpu().numpy().view(np.uint16), ref["out"])
        assert ok.all(), f"{name} combine: {int((~ok).sum())} of {ok.size} elements off"
    return sh, wl, b


def test_full_size_decode():
    sh, wl, b = compare_full_size("decode", full_oracle=True)
    # closed form up to two bf16 roundings: out ~= x * sum_k w_k alpha_k
    x = torch.from_numpy(W.bf16_bits_to_f32(wl.x_bf16)).cuda().double()
    f = torch.from_numpy((wl.weights.astype(np.float64) * wl.alpha[wl.idx]).sum(-1)).cuda()
    want = x * f[..., None]
    got = (b.out.to(torch.int32) & 0xFFFF).to(torch.int32)
    got = (got << 16).view(torch.float32).double()
    nz = want != 0
    rel = ((got - want).abs()[nz] / want.abs()[nz]).max().item()
    assert rel <= 2 * 2.0 ** -8, rel


def test_full_size_decode_zipf():
    compare_full_size("decode_zipf", full_oracle=True)


def _unsign_zero(a):
    """-0 and +0 are the same number: map the bf16 pattern 0x8000 to 0."""
    return a.masked_fill(a == -32768, 0) if isinstance(a, torch.Tensor) else np.where(a == 0x8000, 0, a)


def assert_tokens_equal(got: torch.Tensor, want: np.ndarray, what: str):
    """Equality as numbers of [N][T][H] bf16 tensors (a weighted sum that
    starts from +0 turns -0 inputs into +0), with a readable report."""
    w = _unsign_zero(torch.from_numpy(want.view(np.int16)).to(got.device))
    bad = (_unsign_zero(got) != w)
    if bool(bad.any()):
        tok = bad.any(dim=-1).nonzero().cpu().numpy()
        n_el = int(bad.sum().item())
        g = got.cpu().numpy().view(np.uint16)
        s, t = tok[0]
        h = np.nonzero(g[s, t] != want[s, t])[0][:8]
        raise AssertionError(
            f"{what}: {len(tok)} tokens / {n_el} elements differ; first (s,t)={tuple(tok[0])} "
            f"h={h.tolist()} got={g[s, t][h].tolist()} want={want[s, t][h].tolist()}; "
            f"tokens={tok[:10].tolist()}")


def test_full_size_worst_all_to_rank0():
    sh, wl, b = compare_full_size("worst")
    # identity experts, weights summing to one: every output token equals x
    assert_tokens_equal(b.out, wl.x_bf16, "worst combine")


def test_full_size_prefill_fp8():
    sh, wl, b = compare_full_size("prefill", n_slots=2000, n_tokens=100)
    # identity on dequantised rows: every output token equals bf16(dequant(x))
    N, T, H = sh.n_ranks, sh.tokens, sh.hidden
    want = np.empty((N, T, H), np.uint16)
    for s in range(N):
        for t in range(T):
            want[s, t] = oracle.expert_row([wl.planes[0][s, t], wl.planes[1][s, t]], 0, 1, H, None)
    assert_tokens_equal(b.out, want, "prefill combine")


def test_misaligned_row_buffers_are_rejected():
    sh = W.CONFIGS["tiny"]
    d = desc_of(sh)
    b = ep.Buffers(d)
    raw = torch.empty(b.x[0].numel() + 64, dtype=torch.uint8, device="cuda")
    shifted = raw[8:8 + b.x[0].numel()]                  # 8-byte aligned only
    with pytest.raises(ep.EPError) as e:
        ep.dispatch_pack(d, [shifted], b.plan_ws, b.send)
    assert e.value.code == ep.EP_ERR_INVALID_ARG and "aligned" in str(e.value)
    out_raw = torch.empty(b.out.numel() + 8, dtype=torch.int16, device="cuda")
    with pytest.raises(ep.EPError):
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, out_raw[4:4 + b.out.numel()])
    ws_raw = torch.empty(b.plan_ws.numel() + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ep.EPError) as e:
        ep.plan(d, b.idx, ws_raw[4:4 + b.plan_ws.numel()], b.status)
    assert e.value.code == ep.EP_ERR_INVALID_ARG and "plan_ws" in str(e.value)


def _alloc_range(ptr):
    """(base, size) of the device allocation holding ptr, from the HIP
    runtime torch has loaded."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    rc = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(ptr))
    assert rc == 0, rc
    return base.value, size.value


def test_buffers_smaller_than_the_call_needs_are_rejected():
    """A pointer whose required extent runs past the end of its allocation
    fails validation (nothing is launched)."""
    sh = W.CONFIGS["tiny"]
    d = desc_of(sh)
    b = ep.Buffers(d)
    upload(b, W.make_workload(sh))
    need = d.n_ranks * d.tokens * 2 * d.hidden                  # bytes of out
    base, size = _alloc_range(b.out.data_ptr())
    short = (base + size - need // 2) & ~15
    with pytest.raises(ep.EPError) as e:
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, short)
    assert e.value.code == ep.EP_ERR_INVALID_ARG and "smaller" in str(e.value)
    wbase, wsize = _alloc_range(b.plan_ws.data_ptr())
    short_ws = (wbase + wsize - ep.plan_bytes(d) // 2) & ~15
    with pytest.raises(ep.EPError) as e:
        ep.plan(d, b.idx, short_ws, b.status)
    assert e.value.code == ep.EP_ERR_INVALID_ARG and "plan_ws" in str(e.value)
    ep.plan(d, b.idx, b.plan_ws, b.status)                        # full sizes pass
    torch.cuda.synchronize()

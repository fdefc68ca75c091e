"""Split dispatch (sender half, receiver half, private per-sender regions)
against the unsplit path and the CPU oracle.

Bar: every plan table and every delivered grouped row identical to the
unsplit path (itself bit-exact against the oracle); the rows the sender
half placed in the private regions equal the unsplit send rows they stand
for, and the rest of its send buffer equals the unsplit send buffer.
"""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import (plan_fields, bf16_close, desc_of, expected_plan_extras, note,
                      plan_arrays, run_path, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def run_split(d, b, wl, P, stream=None, between=None):
    """send half -> (optional independent work) -> receive half -> expert -> combine."""
    alpha = torch.from_numpy(wl.alpha).to(b.idx.device) if wl.alpha is not None else None
    priv = ep.priv_buffers(d, P) if P > 0 else []
    b.status.zero_()
    ep.dispatch_send(d, b.idx, b.x, b.plan_ws, b.send, priv, P, b.status, stream)
    if between is not None:
        between()
    ep.dispatch_recv_split(d, b.send, priv, P, b.plan_ws, b.grouped, b.status, stream)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, stream)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, stream)
    return priv


def check_split(sh, wl, P, cap=0):
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    L = E // N
    note(f"split {sh.name} N={N} T={T} H={sh.hidden} E={E} R={R} P={P} cap={cap}")
    ref_b = ep.Buffers(d)
    upload(ref_b, wl)
    run_path(d, ref_b, wl)
    b = ep.Buffers(d)
    upload(b, wl)
    for t in b.send:
        t.zero_()
    priv = run_split(d, b, wl, P)
    torch.cuda.synchronize()
    assert int(b.status.item()) == int(ref_b.status.item())
    got, want = plan_arrays(d, b), plan_arrays(d, ref_b)
    for f in plan_fields(d):
        np.testing.assert_array_equal(got[f], want[f], err_msg=f)
    p = oracle.plan(N, T, E, R, cap, wl.idx)
    assert int(b.status.item()) == p["status"]
    for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    for f, v in expected_plan_extras(p, wl.idx, N, E, cap).items():
        np.testing.assert_array_equal(got[f], v, err_msg=f)
    totals = p["recv_off"][:, N]
    so = p["send_off"]
    for q in range(len(wl.planes)):
        ref_send = ref_b.send[q].cpu().numpy()
        send = b.send[q].cpu().numpy()
        pv = priv[q].cpu().numpy() if P > 0 else None
        for s in range(N):
            for dd in range(N):
                lo, hi = int(so[s, dd * L]), int(so[s, (dd + 1) * L])
                k = min(P, hi - lo)
                if k > 0:
                    np.testing.assert_array_equal(pv[dd, s, :k], ref_send[s, lo:lo + k],
                                                  err_msg=f"priv {dd}<-{s}")
                np.testing.assert_array_equal(send[s, lo + k:hi], ref_send[s, lo + k:hi],
                                              err_msg=f"send {s}->{dd}")
        grouped, ref_g = b.grouped[q].cpu().numpy(), ref_b.grouped[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(grouped[dd, :n], ref_g[dd, :n], err_msg=f"grouped {dd}")
    out, ref_out = b.out.cpu().numpy(), ref_b.out.cpu().numpy()
    np.testing.assert_array_equal(out, ref_out)
    return d, b


SPLIT_SHAPES = [
    (W.CONFIGS["tiny"], 0), (W.CONFIGS["tiny"], 1), (W.CONFIGS["tiny"], 3),
    (W.CONFIGS["tiny"], 32), (W.CONFIGS["tiny_zipf"], 2),
    (W.Shape("single_rank", 1, 37, 64, 5, 2), 4),
    (W.Shape("topk1", 4, 50, 128, 8, 1), 5),
    (W.Shape("rank0_repeated_ids", 8, 8, 64, 32, 8, routing="rank0"), 7),
    (W.Shape("multi_chunk_plan", 2, 3000, 64, 12, 3, expert="scale"), 100),
    (W.Shape("ragged_row", 3, 7, 1000, 6, 2, expert="scale"), 2),
    (W.Shape("fp8_h1024", 4, 12, 1024, 16, 4, payload=W.PAYLOAD_FP8_B128, expert="dequant"), 3),
    (W.Shape("max_experts", 2, 64, 64, 2048, 16), 9),
    (W.Shape("many_ranks", 128, 4, 64, 128, 4, routing="zipf"), 1),
    (W.Shape("no_tokens", 2, 0, 64, 4, 2), 0),
    (W.Shape("large_source", 2, 512, 4608, 16, 8), 5),           # windowed split sender
    (W.Shape("huge_source", 2, 4200, 4096, 16, 4), 3),           # token-order split sender
]


@pytest.mark.parametrize("sh,P", SPLIT_SHAPES, ids=[f"{s.name}-P{P}" for s, P in SPLIT_SHAPES])
def test_split_equals_unsplit(sh, P):
    check_split(sh, W.make_workload(sh), P)


def test_split_bad_ids_and_capacity():
    sh = W.Shape("bad_tight", 4, 32, 128, 16, 3, routing="zipf", expert="scale", seed=12)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    idx[0, 0, 0] = 16
    idx[2, 7, 1] = -1
    wl = W.make_workload(sh, idx=idx)
    full = oracle.plan(4, 32, 16, 3, oracle.recv_bound(4, 32, 16, 3), wl.idx)
    cap = int(full["recv_off"][:, 4].max()) - 5
    d, b = check_split(sh, wl, 3, cap=cap)
    assert int(b.status.item()) == ep.EP_STATUS_BAD_EXPERT | ep.EP_STATUS_CAPACITY


def test_split_windowed_sender_with_bad_ids_and_tight_capacity():
    """The windowed sender with private regions: dropped slots leave gaps in
    the window lists, and rows past a tight capacity are dropped on the
    receive side."""
    sh = W.Shape("window_bad_split", 2, 600, 4608, 16, 8, expert="scale", seed=5)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    rng = np.random.default_rng(8)
    bad = rng.random(idx.shape) < 0.02
    idx[bad] = rng.choice([-1, 16, 99], size=int(bad.sum()))
    wl = W.make_workload(sh, idx=idx)
    full = oracle.plan(2, 600, 16, 8, oracle.recv_bound(2, 600, 16, 8), idx)
    cap = int(full["recv_off"][:, 2].max()) - 3
    d, b = check_split(sh, wl, 5, cap=cap)
    assert int(b.status.item()) == ep.EP_STATUS_BAD_EXPERT | ep.EP_STATUS_CAPACITY


def test_independent_work_between_halves_on_another_stream():
    """The sender half on stream A, a GEMM that does not depend on it on
    stream B while A goes on to the receiver half: same results."""
    sh = W.CONFIGS["tiny_zipf"]
    wl = W.make_workload(sh)
    d = desc_of(sh)
    ref_b = ep.Buffers(d)
    upload(ref_b, wl)
    run_path(d, ref_b, wl)
    a = torch.randn(1024, 1024, device="cuda")
    c_ref = a @ a
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    b = ep.Buffers(d)
    with torch.cuda.stream(sa):
        upload(b, wl)
    sa.synchronize()
    res = {}

    def between():
        with torch.cuda.stream(sb):
            res["c"] = a @ a

    run_split(d, b, wl, 2, stream=sa, between=between)
    torch.cuda.synchronize()
    for f in plan_fields(d):
        np.testing.assert_array_equal(plan_arrays(d, b)[f], plan_arrays(d, ref_b)[f], err_msg=f)
    assert torch.equal(b.out, ref_b.out)
    assert torch.equal(res["c"], c_ref)


def test_two_micro_batches_interleaved():
    """send(A), send(B), receive(A), receive(B) with separate workspaces."""
    shs = [W.CONFIGS["tiny"], W.Shape("tiny_b", 4, 16, 256, 16, 2, routing="zipf", seed=9)]
    wls = [W.make_workload(sh) for sh in shs]
    d = desc_of(shs[0])
    refs, bs, privs = [], [], []
    for wl in wls:
        rb = ep.Buffers(d)
        upload(rb, wl)
        run_path(d, rb, wl)
        refs.append(rb)
        b = ep.Buffers(d)
        upload(b, wl)
        b.status.zero_()
        bs.append(b)
        privs.append(ep.priv_buffers(d, 2))
    for b, pv in zip(bs, privs):
        ep.dispatch_send(d, b.idx, b.x, b.plan_ws, b.send, pv, 2, b.status)
    for b, pv in zip(bs, privs):
        ep.dispatch_recv_split(d, b.send, pv, 2, b.plan_ws, b.grouped, b.status)
        ep.expert_stub(d, b.grouped, None, b.plan_ws, b.expert_out)
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    torch.cuda.synchronize()
    for b, rb in zip(bs, refs):
        assert int(b.status.item()) == 0
        for f in plan_fields(d):
            np.testing.assert_array_equal(plan_arrays(d, b)[f], plan_arrays(d, rb)[f], err_msg=f)
        assert torch.equal(b.out, rb.out)


def test_split_rejects_bad_private_rows():
    sh = W.CONFIGS["tiny"]
    d = desc_of(sh)
    b = ep.Buffers(d)
    for P in (-1, sh.tokens * sh.topk + 1):
        with pytest.raises(ep.EPError) as e:
            ep.dispatch_send(d, b.idx, b.x, b.plan_ws, b.send, [], P, b.status)
        assert e.value.code == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EPError) as e:
        ep.dispatch_recv_split(d, b.send, [], 2, b.plan_ws, b.grouped, b.status)
    assert e.value.code == ep.EP_ERR_INVALID_ARG


@pytest.mark.parametrize("name,P", [("decode", 4), ("decode_fp8", 2), ("worst", 16)])
def test_split_full_size(name, P):
    """Full-size workloads: plan tables and grouped layout identical to the
    unsplit path, on the device."""
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    d = desc_of(sh)
    cap = ep.capacity(d)
    N = sh.n_ranks
    note(f"split full-size {name} P={P}")
    b = ep.Buffers(d)
    upload(b, wl)
    run_path(d, b, wl)
    torch.cuda.synchronize()
    want = plan_arrays(d, b)
    totals = want["recv_off"][:, N]
    rows = [min(int(totals[dd]), cap) for dd in range(N)]
    ref_grouped = [[g[dd, :rows[dd]].clone() for dd in range(N)] for g in b.grouped]
    ref_out = b.out.clone()
    b.plan_ws.zero_()
    for g in b.grouped:
        for dd in range(N):
            g[dd, :rows[dd]].zero_()
    run_split(d, b, wl, P)
    torch.cuda.synchronize()
    assert int(b.status.item()) == 0
    got = plan_arrays(d, b)
    for f in plan_fields(d):
        np.testing.assert_array_equal(got[f], want[f], err_msg=f)
    for g, rg in zip(b.grouped, ref_grouped):
        for dd in range(N):
            assert torch.equal(g[dd, :rows[dd]], rg[dd]), f"grouped {dd}"
    assert torch.equal(b.out, ref_out)


def run_overlapped(d, b, wl, P, sa, sb):
    """send_plan on stream A; the exchange (recv_plan) on stream B while A
    packs; the pull after both."""
    priv = ep.priv_buffers(d, P) if P > 0 else []
    alpha = torch.from_numpy(wl.alpha).to(b.idx.device) if wl.alpha is not None else None
    b.status.zero_()
    torch.cuda.synchronize()
    ep.dispatch_send_plan(d, b.idx, b.plan_ws, b.status, sa)
    counts_ready = torch.cuda.Event()
    counts_ready.record(sa)
    sb.wait_event(counts_ready)
    ep.dispatch_recv_plan(d, b.plan_ws, b.status, sb)
    offsets_ready = torch.cuda.Event()
    offsets_ready.record(sb)
    ep.dispatch_send_pack(d, b.idx, b.x, b.plan_ws, b.send, priv, P, sa)
    sa.wait_event(offsets_ready)
    ep.dispatch_recv_pull(d, b.send, priv, P, b.plan_ws, b.grouped, sa)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sa)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sa)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,P", [("tiny", 0), ("tiny_zipf", 3), ("decode", 0), ("decode", 4),
                                    ("worst", 2)])
def test_exchange_overlapped_with_pack_equals_unsplit(name, P):
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    d = desc_of(sh)
    N = sh.n_ranks
    cap = ep.capacity(d)
    note(f"split overlapped {name} P={P}")
    ref = ep.Buffers(d)
    upload(ref, wl)
    run_path(d, ref, wl)
    torch.cuda.synchronize()
    want = plan_arrays(d, ref)
    totals = want["recv_off"][:, N]
    rows = [min(int(totals[dd]), cap) for dd in range(N)]
    ref_grouped = [[g[dd, :rows[dd]].clone() for dd in range(N)] for g in ref.grouped]
    ref_out = ref.out.clone()
    del ref
    gc.collect()
    b = ep.Buffers(d)
    upload(b, wl)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    run_overlapped(d, b, wl, P, sa, sb)
    assert int(b.status.item()) == 0
    got = plan_arrays(d, b)
    for f in plan_fields(d):
        np.testing.assert_array_equal(got[f], want[f], err_msg=f)
    for g, rg in zip(b.grouped, ref_grouped):
        for dd in range(N):
            assert torch.equal(g[dd, :rows[dd]], rg[dd]), f"grouped {dd}"
    assert torch.equal(b.out, ref_out)


def test_split_pieces_validate_before_enqueueing():
    sh = W.CONFIGS["tiny"]
    d = desc_of(sh)
    b = ep.Buffers(d)
    with pytest.raises(ep.EPError):
        ep.dispatch_send(d, b.idx, b.x, b.plan_ws, [None], [], 0, b.status)   # null send plane
    with pytest.raises(ep.EPError):
        ep.dispatch_recv_pull(d, b.send, [], 1, b.plan_ws, b.grouped)          # P > 0, no priv

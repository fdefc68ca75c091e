"""ep_dispatch (plan + pack + receive in one call) against the three calls
it replaces: every plan table, every send row, every delivered grouped row
and the status word must be identical; small cases also against the oracle."""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import plan_fields, desc_of, expected_plan_extras, note, plan_arrays, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _three_calls(d, b):
    b.status.zero_()
    ep.plan(d, b.idx, b.plan_ws, b.status)
    ep.dispatch_pack(d, b.x, b.plan_ws, b.send)
    ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped)
    torch.cuda.synchronize()


def compare(sh, wl, cap=0, with_oracle=True):
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    N = sh.n_ranks
    note(f"dispatch {sh.name} N={N} T={sh.tokens} H={sh.hidden} E={sh.n_experts} R={sh.topk}")
    ref = ep.Buffers(d)
    upload(ref, wl)
    _three_calls(d, ref)
    want = plan_arrays(d, ref)
    totals = want["recv_off"][:, N]
    rows = [min(int(totals[dd]), cap) for dd in range(N)]
    ref_send = [t.clone() for t in ref.send]
    ref_grouped = [[g[dd, :rows[dd]].clone() for dd in range(N)] for g in ref.grouped]
    ref_status = int(ref.status.item())
    del ref
    gc.collect()
    b = ep.Buffers(d)
    upload(b, wl)
    b.plan_ws.fill_(0x5A)                      # stale workspace bytes must not matter
    b.status.zero_()
    ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status)
    torch.cuda.synchronize()
    assert int(b.status.item()) == ref_status
    got = plan_arrays(d, b)
    for f in plan_fields(d):
        np.testing.assert_array_equal(got[f], want[f], err_msg=f)
    so = want["send_off"]
    for q, (t, rt) in enumerate(zip(b.send, ref_send)):
        for s in range(N):
            n = int(so[s, -1])
            assert torch.equal(t[s, :n], rt[s, :n]), f"send plane {q} rank {s}"
    for g, rg in zip(b.grouped, ref_grouped):
        for dd in range(N):
            assert torch.equal(g[dd, :rows[dd]], rg[dd]), f"grouped {dd}"
    if with_oracle:
        p = oracle.plan(N, sh.tokens, sh.n_experts, sh.topk, cap, wl.idx)
        for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
            np.testing.assert_array_equal(got[f], p[f], err_msg=f)
        for f, v in expected_plan_extras(p, wl.idx, N, sh.n_experts, cap).items():
            np.testing.assert_array_equal(got[f], v, err_msg=f)
    return b


SHAPES = [
    W.CONFIGS["tiny"], W.CONFIGS["tiny_zipf"],
    W.Shape("single_rank", 1, 37, 64, 5, 2),
    W.Shape("topk1", 4, 50, 128, 8, 1),
    W.Shape("rank0_repeated_ids", 8, 8, 64, 32, 8, routing="rank0"),
    W.Shape("chunk_exactly_full", 4, 512, 256, 32, 8),           # T R = 4096
    W.Shape("over_one_chunk", 2, 513, 256, 32, 8),                # T R = 4104: three calls
    W.Shape("e512", 4, 40, 256, 512, 6, routing="zipf", seed=3),
    W.Shape("e1024_three_calls", 4, 40, 256, 1024, 6, seed=4),
    W.Shape("ragged_row", 3, 7, 1000, 6, 2, expert="scale"),
    W.Shape("wide_row", 2, 5, 8192, 4, 2),
    W.Shape("fp8_h1024", 4, 12, 1024, 16, 4, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("fp8_h7168", 4, 12, 7168, 16, 4, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("many_ranks", 128, 4, 64, 128, 4, routing="zipf"),
    W.Shape("no_tokens", 2, 0, 64, 4, 2),
    # 4 to 32 MiB of token rows per source: the windowed sender with the
    # exchange folded in (T R = 4096), and in the three-call form; over
    # 32 MiB the token-order sender with the exchange folded in
    W.Shape("large_source_exchange", 2, 512, 4608, 16, 8),
    W.Shape("large_source_fp8", 2, 600, 7168, 16, 8, payload=W.PAYLOAD_FP8_B128, expert="dequant"),
    W.Shape("huge_source_exchange", 2, 4096, 4160, 4, 1),
]


@pytest.mark.parametrize("sh", SHAPES, ids=[s.name for s in SHAPES])
def test_dispatch_equals_three_calls(sh):
    compare(sh, W.make_workload(sh))


def test_dispatch_bad_ids_and_capacity():
    sh = W.Shape("bad_tight", 4, 32, 128, 16, 3, routing="zipf", expert="scale", seed=12)
    wl = W.make_workload(sh)
    idx = wl.idx.copy()
    idx[0, 0, 0] = 16
    idx[1, 5, 2] = -3
    wl = W.make_workload(sh, idx=idx)
    full = oracle.plan(4, 32, 16, 3, oracle.recv_bound(4, 32, 16, 3), wl.idx)
    cap = int(full["recv_off"][:, 4].max()) - 5
    b = compare(sh, wl, cap=cap)
    assert int(b.status.item()) == ep.EP_STATUS_BAD_EXPERT | ep.EP_STATUS_CAPACITY


@pytest.mark.parametrize("name", ["decode", "decode_zipf", "decode_fp8", "worst"])
def test_dispatch_full_size(name):
    """The benchmarked one-call dispatch at full size: equal to the three
    calls, its plan tables equal to the oracle's, and every send row and
    delivered grouped row equal to the token row the oracle's plan puts
    there (compared on the device)."""
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    b = compare(sh, wl)
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    p = oracle.plan(N, T, E, R, ep.capacity(b.desc), wl.idx)
    ss, tt, _ = np.unravel_index(np.arange(N * T * R), (N, T, R))
    dd = wl.idx.reshape(-1) // (E // N)
    for q in range(len(wl.planes)):
        for lo in range(0, N * T * R, 8192):
            sl = slice(lo, min(lo + 8192, N * T * R))
            si = torch.from_numpy(ss[sl]).cuda()
            ti = torch.from_numpy(tt[sl]).cuda()
            want = b.x[q][si, ti]
            spi = torch.from_numpy(p["send_pos"].reshape(-1)[sl].astype(np.int64)).cuda()
            gpi = torch.from_numpy(p["grp_pos"].reshape(-1)[sl].astype(np.int64)).cuda()
            di = torch.from_numpy(dd[sl].astype(np.int64)).cuda()
            assert torch.equal(b.send[q][si, spi], want), f"send rows {lo}.."
            assert torch.equal(b.grouped[q][di, gpi], want), f"grouped rows {lo}.."

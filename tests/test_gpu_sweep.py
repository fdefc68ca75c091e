"""Seeded sweep of random small shapes through the one-call dispatch, the
stand-in expert, combine and the partial-sum combine, against the oracle:
random N, experts per rank, R (including R > E / N with repeated ids), T
(including 0), H, payload, invalid ids and tight capacities. Each case also
runs the staged receive (transfer, then unpack) and the split dispatch with
a random number of private rows. A second sweep runs the quantising
dispatch (bf16 rows in) over random shapes and value ranges."""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import bf16_close, desc_of, expected_plan_extras, note, plan_arrays, upload

pytestmark = pytest.mark.gpu

CASES = 40


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 17))
    L = int(rng.integers(1, 9))
    E = N * L
    R = int(rng.integers(1, 13))
    T = int(rng.choice([0, 1, 3, 17, 64, 129, 300]))
    fp8 = bool(rng.random() < 0.3)
    H = int(rng.choice([128, 256, 1024])) if fp8 else int(rng.choice([8, 64, 136, 1000, 2048]))
    sh = W.Shape(f"sweep{seed}", N, T, H, E, R, payload=W.PAYLOAD_FP8_B128 if fp8 else W.PAYLOAD_BF16,
                 expert="dequant" if fp8 else "scale", seed=seed)
    idx = rng.integers(0, E, size=(N, T, R)).astype(np.int32)   # repeats allowed
    if rng.random() < 0.3 and idx.size:
        bad = rng.random(idx.shape) < 0.05
        idx[bad] = rng.choice([-1, E, E + 7], size=int(bad.sum()))
    wl = W.make_workload(sh, idx=idx)
    cap = 0
    if rng.random() < 0.3 and idx.size:
        full = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), idx)
        cap = max(1, int(full["recv_off"][:, N].max()) - int(rng.integers(0, 4)))
    return sh, wl, cap


@pytest.mark.parametrize("seed", range(CASES))
def test_sweep_against_oracle(seed):
    sh, wl, cap = draw_case(seed)
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    N = sh.n_ranks
    note(f"sweep {seed}: N={N} T={sh.tokens} H={sh.hidden} E={sh.n_experts} R={sh.topk} "
         f"payload={sh.payload} cap={cap}")
    b = ep.Buffers(d)
    upload(b, wl)
    alpha = torch.from_numpy(wl.alpha).cuda() if wl.alpha is not None else None
    b.status.zero_()
    ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    partial = torch.zeros((N, sh.tokens * sh.topk, sh.hidden), dtype=torch.int16, device="cuda")
    pout = torch.zeros_like(b.out)
    ep.combine_presum(d, b.expert_out, b.weights, b.plan_ws, partial, pout)
    torch.cuda.synchronize()
    ref = oracle.run(wl, cap=cap)
    p = ref["plan"]
    assert int(b.status.item()) == p["status"]
    got = plan_arrays(d, b)
    for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    for f, v in expected_plan_extras(p, wl.idx, N, sh.n_experts, cap).items():
        np.testing.assert_array_equal(got[f], v, err_msg=f)
    totals = p["recv_off"][:, N]
    for q in range(len(wl.planes)):
        g = b.grouped[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(g[dd, :n], ref["grouped"][q][dd, :n])
    out = b.out.cpu().numpy().view(np.uint16)
    assert bf16_close(out, ref["out"]).all()
    want_partial, want_out = oracle.combine_presum(ref["y"], wl.weights, wl.idx, p)
    np.testing.assert_array_equal(pout.cpu().numpy().view(np.uint16), want_out)

    # staged receive: the receive buffers as the oracle's per-pair write; the
    # grouped layout too unless capacity overflowed (rows past cap never
    # reach a receive buffer)
    recv = [torch.zeros((N, cap, t.shape[2]), dtype=torch.uint8, device="cuda") for t in b.send]
    staged = [torch.zeros_like(g) for g in b.grouped]
    ep.dispatch_transfer(d, b.send, b.plan_ws, recv)
    ep.dispatch_unpack(d, recv, b.plan_ws, staged)
    torch.cuda.synchronize()
    for q in range(len(wl.planes)):
        rv, sg = recv[q].cpu().numpy(), staged[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(rv[dd, :n], ref["recv"][q][dd, :n], err_msg=f"recv {dd}")
            if not p["status"] & 2:
                np.testing.assert_array_equal(sg[dd, :n], ref["grouped"][q][dd, :n],
                                              err_msg=f"staged grouped {dd}")
    del recv, staged

    # split dispatch with P private rows per (destination, source)
    P = min(int(np.random.default_rng(2000 + seed).integers(0, 6)), sh.tokens * sh.topk)
    ws2 = torch.empty_like(b.plan_ws)
    send2 = [torch.zeros_like(t) for t in b.send]
    grouped2 = [torch.zeros_like(g) for g in b.grouped]
    priv = ep.priv_buffers(d, P)
    st2 = torch.zeros_like(b.status)
    ep.dispatch_send(d, b.idx, b.x, ws2, send2, priv, P, st2)
    ep.dispatch_recv_split(d, send2, priv, P, ws2, grouped2, st2)
    torch.cuda.synchronize()
    assert int(st2.item()) == p["status"]
    for q in range(len(wl.planes)):
        g2 = grouped2[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(g2[dd, :n], ref["grouped"][q][dd, :n],
                                          err_msg=f"split P={P} grouped {dd}")
    np.testing.assert_array_equal(partial.cpu().numpy().view(np.uint16), want_partial)
    del b
    gc.collect()


QUANT_CASES = 30


def draw_quant_case(seed):
    """A random shape for the quantising dispatch: block-fp8 payload, H a
    multiple of 128 (above 8192 the wave-per-segment sender runs), token
    values over a random dynamic range per block, sometimes exact zeros,
    invalid ids and a tight capacity."""
    rng = np.random.default_rng(5000 + seed)
    N = int(rng.integers(1, 13))
    L = int(rng.integers(1, 9))
    E = N * L
    R = int(rng.integers(1, 10))
    T = int(rng.choice([0, 1, 5, 33, 130]))
    H = 128 * int(rng.choice([1, 2, 7, 8, 56, 65, 72]))
    if H > 4096:
        T = min(T, 33)                 # keeps the CPU side of each case to about a second
    sh = W.Shape(f"qsweep{seed}", N, T, H, E, R, payload=W.PAYLOAD_FP8_B128, expert="dequant",
                 seed=seed)
    idx = np.stack([np.argsort(rng.random((N, T, E)), axis=-1)[..., k % E] for k in range(R)],
                   axis=-1).astype(np.int32) if T else np.zeros((N, 0, R), np.int32)
    if rng.random() < 0.3 and idx.size:
        bad = rng.random(idx.shape) < 0.05
        idx[bad] = rng.choice([-1, E, E + 3], size=int(bad.sum()))
    wl = W.make_workload(sh, idx=idx)
    x = W.bf16_bits_to_f32(wl.x_bf16).astype(np.float64).reshape(-1, 128)
    if x.size:
        x *= np.exp2(rng.integers(-40, 40, size=(x.shape[0], 1)).astype(np.float64))
        x[rng.random(x.shape) < 0.02] = 0.0
    wl.x_bf16 = W.to_bf16_bits(x.astype(np.float32).reshape(wl.x_bf16.shape))
    codes, scales = oracle.quantize_b128(wl.x_bf16)
    wl.planes = [codes, scales.view(np.uint8)]
    cap = 0
    if rng.random() < 0.3 and idx.size:
        full = oracle.plan(N, T, E, R, oracle.recv_bound(N, T, E, R), idx)
        cap = max(1, int(full["recv_off"][:, N].max()) - int(rng.integers(0, 4)))
    return sh, wl, cap


@pytest.mark.parametrize("seed", range(QUANT_CASES))
def test_quant_sweep_against_oracle(seed):
    """ep_dispatch_quant (bf16 rows in, the sender quantises), the
    dequantising stand-in expert and combine, against the oracle: status,
    plan tables, filled send rows, delivered grouped rows and expert rows bit
    for bit, the output within the combine bar."""
    sh, wl, cap = draw_quant_case(seed)
    d = desc_of(sh, cap)
    cap = ep.capacity(d)
    N, T, R = sh.n_ranks, sh.tokens, sh.topk
    note(f"quant sweep {seed}: N={N} T={T} H={sh.hidden} E={sh.n_experts} R={R} cap={cap}")
    b = ep.Buffers(d)
    upload(b, wl)
    x = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda()
    b.status.zero_()
    ep.dispatch_quant(d, b.idx, x, b.plan_ws, b.send, b.grouped, b.status)
    ep.expert_stub(d, b.grouped, None, b.plan_ws, b.expert_out)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    torch.cuda.synchronize()
    ref = oracle.run(wl, cap=cap)
    p = ref["plan"]
    assert int(b.status.item()) == p["status"]
    got = plan_arrays(d, b)
    for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
        np.testing.assert_array_equal(got[f], p[f], err_msg=f)
    oc, osc = oracle.dispatch_pack_quant(wl.x_bf16, p)
    filled = p["send_off"][:, -1]
    sc = b.send[0].cpu().numpy()
    ss = b.send[1].cpu().numpy().view(np.uint32)
    for s in range(N):
        n = int(filled[s])
        np.testing.assert_array_equal(sc[s, :n], oc[s, :n], err_msg=f"codes {s}")
        np.testing.assert_array_equal(ss[s, :n], osc.view(np.uint32)[s, :n], err_msg=f"scales {s}")
    totals = p["recv_off"][:, N]
    y = b.expert_out.cpu().numpy().view(np.uint16)
    for q in range(2):
        g = b.grouped[q].cpu().numpy()
        for dd in range(N):
            n = min(int(totals[dd]), cap)
            np.testing.assert_array_equal(g[dd, :n], ref["grouped"][q][dd, :n])
    for dd in range(N):
        n = min(int(totals[dd]), cap)
        np.testing.assert_array_equal(y[dd, :n], ref["y"][dd, :n])
    out = b.out.cpu().numpy().view(np.uint16)
    assert bf16_close(out, ref["out"]).all()

"""Helpers for the GPU tests: run the library on a workload, read results."""
from __future__ import annotations

import sys

import numpy as np
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W

PLAN_FIELDS = ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos",
               "src_off", "comb_row", "grp_slot", "send_slot", "recv_rows", "send_seg",
               "win_list")


def note(msg: str) -> None:
    """Name the case before any GPU step (a fault can end the process)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def desc_of(sh: W.Shape, cap: int = 0) -> ep.Desc:
    return ep.make_desc(sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk,
                        sh.payload, cap or sh.cap_rows)


def upload(b: ep.Buffers, wl: W.Workload) -> None:
    b.idx.copy_(torch.from_numpy(wl.idx))
    b.weights.copy_(torch.from_numpy(wl.weights))
    for q, plane in enumerate(wl.planes):
        b.x[q].copy_(torch.from_numpy(plane))


def run_path(d: ep.Desc, b: ep.Buffers, wl: W.Workload, staged: bool = False,
             stream=None) -> None:
    """plan -> pack -> (recv | transfer + unpack) -> stand-in expert -> combine."""
    alpha = torch.from_numpy(wl.alpha).to(b.idx.device) if wl.alpha is not None else None
    b.status.zero_()
    ep.plan(d, b.idx, b.plan_ws, b.status, stream)
    ep.dispatch_pack(d, b.x, b.plan_ws, b.send, stream)
    if staged:
        ep.dispatch_transfer(d, b.send, b.plan_ws, b.recv, stream)
        ep.dispatch_unpack(d, b.recv, b.plan_ws, b.grouped, stream)
    else:
        ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, stream)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, stream)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, stream)


def window_of(N: int, T: int, R: int, tok_bytes: int):
    """(W, nwin) of the windowed sender, by the rule the header states:
    (0, 0) unless one source's token rows take more than 4 and at most
    32 MiB and all send buffers at most 2 GiB; W is the largest power of two
    with W * tok_bytes <= 4 MiB."""
    src = T * tok_bytes
    if not (4 << 20 < src <= 32 << 20) or N * T * R * tok_bytes > 2 << 30:
        return 0, 0
    w = 1
    while 2 * w * tok_bytes <= 4 << 20:
        w *= 2
    return w, -(-T // w)


def tok_bytes_of(d: ep.Desc) -> int:
    return sum(ep.row_bytes(d, q) for q in range(ep.num_planes(d)))


def expected_win_list(p: dict, N: int, T: int, R: int, tok_bytes: int):
    """The windowed sender's work list from the oracle's send positions: per
    window of W tokens, its slots in send-row order as (send row, token),
    then (-1, -1); None when the sender is not windowed."""
    W, nwin = window_of(N, T, R, tok_bytes)
    if W == 0:
        return None
    TR = T * R
    out = np.full((N, nwin, W * R, 2), -1, np.int64)
    sp = p["send_pos"].reshape(N, TR).astype(np.int64)
    for s in range(N):
        for w in range(nwin):
            lo, hi = w * W * R, min(TR, (w + 1) * W * R)
            i = np.arange(lo, hi)
            pos = sp[s, lo:hi]
            ok = pos >= 0
            i, pos = i[ok], pos[ok]
            order = np.argsort(pos, kind="stable")
            out[s, w, :len(order), 0] = s * TR + pos[order]
            out[s, w, :len(order), 1] = s * T + i[order] // R
    return out.reshape(-1, 2).astype(np.int32)


def plan_fields(d: ep.Desc) -> tuple:
    """The plan tables a descriptor has (the windowed list only when used)."""
    if window_of(d.n_ranks, d.tokens, d.topk, tok_bytes_of(d))[0]:
        return PLAN_FIELDS
    return tuple(f for f in PLAN_FIELDS if f != "win_list")


def plan_arrays(d: ep.Desc, b: ep.Buffers) -> dict:
    """Copy every plan table of the workspace to host numpy arrays (the
    windowed sender's list only when the descriptor has one)."""
    N, T, E, R = d.n_ranks, d.tokens, d.n_experts, d.topk
    L = E // N
    shapes = {"cnt": (N, E), "send_off": (N, E + 1), "send_pos": (N, T, R),
              "recv_off": (N, N + 1), "grp_off": (N, L + 1), "grp_pos": (N, T, R),
              "src_off": (N, E), "comb_row": (N, T, R), "grp_slot": (N * T * R,),
              "send_slot": (N, T * R), "recv_rows": (N * T * R, 2), "send_seg": (N, T * R)}
    W, nwin = window_of(N, T, R, tok_bytes_of(d))
    shapes["win_list"] = (N * nwin * W * R, 2)
    v = ep.plan_views(d, b.plan_ws)
    base = b.plan_ws.data_ptr()
    ws = b.plan_ws.cpu().numpy()
    out = {}
    for f in PLAN_FIELDS:
        if getattr(v, f) is None:
            continue
        off = getattr(v, f) - base
        n = int(np.prod(shapes[f]))
        out[f] = ws[off:off + 4 * n].view(np.int32).reshape(shapes[f]).copy()
    return out


def expected_plan_extras(p: dict, idx: np.ndarray, N: int, E: int, cap: int) -> dict:
    """src_off, comb_row, grp_slot, send_slot, recv_rows and send_seg from
    the oracle's cnt, grp_pos, send_pos and send_off and the routing ids, by
    their definitions."""
    L = E // N
    cnt = p["cnt"].astype(np.int64)
    src_off = np.vstack([np.zeros((1, E), np.int64), np.cumsum(cnt, axis=0)[:-1]])
    comb = np.where(p["grp_pos"] >= 0, (idx // L).astype(np.int64) * cap + p["grp_pos"], -1)
    # receive order: rank 0's delivered grouped rows, then rank 1's, ...
    delivered = np.minimum(p["recv_off"][:, N].astype(np.int64), cap)
    dstart = np.concatenate([[0], np.cumsum(delivered)])
    grp_slot = np.full(idx.size, -1, np.int64)
    gp = p["grp_pos"].reshape(-1)
    dd = (idx.reshape(-1) // L)
    ok = gp >= 0
    grp_slot[dstart[dd[ok]] + gp[ok]] = np.nonzero(ok)[0]
    # send_slot: the inverse of send_pos per source, -1 past the filled rows
    T, R = idx.shape[1], idx.shape[2]
    send_slot = np.full((N, T * R), -1, np.int64)
    sp = p["send_pos"].reshape(N, T * R)
    for s in range(N):
        have = sp[s] >= 0
        send_slot[s, sp[s][have]] = s * T * R + np.nonzero(have)[0]
    # recv_rows: (send row, grouped row) of each receive-order entry
    recv_rows = np.full((idx.size, 2), -1, np.int64)
    have = grp_slot >= 0
    gs = grp_slot[have]
    recv_rows[have, 0] = (gs // (T * R)) * T * R + sp.reshape(-1)[gs]
    recv_rows[have, 1] = comb.reshape(-1)[gs]
    # send_seg: destination rank and index inside the segment s -> d
    send_seg = np.full((N, T * R), -1, np.int64)
    ids = idx.reshape(N, T * R).astype(np.int64)
    for s in range(N):
        n = int(p["send_off"][s, E])
        dd = ids[s, send_slot[s, :n] - s * T * R] // L
        send_seg[s, :n] = dd * T * R + (np.arange(n) - p["send_off"][s, dd * L])
    return {"src_off": src_off.astype(np.int32), "comb_row": comb.astype(np.int32),
            "grp_slot": grp_slot.astype(np.int32), "send_slot": send_slot.astype(np.int32),
            "recv_rows": recv_rows.astype(np.int32), "send_seg": send_seg.astype(np.int32)}


def bf16_close(got: np.ndarray, want: np.ndarray, rel: float = 8e-3) -> np.ndarray:
    """Per element: |g - o| <= rel * |o| (so o == 0 requires g == 0)."""
    g = W.bf16_bits_to_f32(got).astype(np.float64)
    o = W.bf16_bits_to_f32(want).astype(np.float64)
    return np.abs(g - o) <= rel * np.abs(o)


def random_bf16(rng: np.random.Generator, shape, lo: int = -6, hi: int = 6) -> np.ndarray:
    """bf16 bit patterns of random sign, exponent in [lo, hi], any mantissa:
    expert rows whose terms cancel, as a grouped GEMM's outputs do."""
    sign = rng.integers(0, 2, shape, dtype=np.uint32) << 15
    expo = rng.integers(127 + lo, 127 + hi + 1, shape, dtype=np.uint32) << 7
    mant = rng.integers(0, 128, shape, dtype=np.uint32)
    return (sign | expo | mant).astype(np.uint16)


def abs_term_sum(weights: np.ndarray, y_slots: np.ndarray) -> np.ndarray:
    """sum_k |w_k| * |y_k| per output element, in float64: weights [..., R]
    fp32, y_slots [..., R, H] bf16 bits of each slot's expert row (zero rows
    for dropped slots). Returns [..., H]."""
    w = np.abs(weights.astype(np.float64))
    out = np.zeros(y_slots.shape[:-2] + y_slots.shape[-1:], np.float64)
    for k in range(y_slots.shape[-2]):
        out += w[..., k, None] * np.abs(W.bf16_bits_to_f32(y_slots[..., k, :]).astype(np.float64))
    return out


def combine_close(got: np.ndarray, want: np.ndarray, abs_sum: np.ndarray, R: int) -> np.ndarray:
    """The combine's bar where the R terms may cancel:
    |g - o| <= 8e-3 |o| + 2 R 2^-24 sum_k |w_k y_k| + 2^-133.
    g sums in fp32 with one rounding per fused multiply-add (error at most
    R 2^-24 sum_k |w_k y_k|), the oracle rounds the exact sum once; both then
    round to bf16 (half an ulp, at most 2^-8 relative each, which the 8e-3
    relative term covers) and 2^-133, the bf16 subnormal step, covers
    results in the subnormal range. With terms of one sign the absolute part
    is far below one ulp of |o| and the bar is the relative one."""
    g = W.bf16_bits_to_f32(got).astype(np.float64)
    o = W.bf16_bits_to_f32(want).astype(np.float64)
    return np.abs(g - o) <= 8e-3 * np.abs(o) + 2.0 * R * 2.0 ** -24 * abs_sum + 2.0 ** -133


def rows_of(t: torch.Tensor, d_idx: np.ndarray, r_idx: np.ndarray) -> np.ndarray:
    """Gather rows t[d, r] on the device, return them on the host."""
    dd = torch.from_numpy(d_idx.astype(np.int64)).to(t.device)
    rr = torch.from_numpy(r_idx.astype(np.int64)).to(t.device)
    return t[dd, rr].cpu().numpy()

#!/usr/bin/env python3
"""Benchmark: one MoE dispatch + combine step of the whole EP group on one GPU.

A step is ep_dispatch (plan, pack and receive) -> ep_combine over the
decode-scale workload (N=32 virtual ranks x T=128 tokens, H=7168 bf16, E=256
experts, top-8 uniform routing, softmax weights); fp8 workloads use
ep_dispatch_quant (the sender quantises bf16 rows). The stand-in expert
(per-expert scale) runs once before timing; its output is what combine
reads in every timed step, so no expert work is inside the timed region.

Prints one JSON line. `value` is the effective HBM throughput of the step:
the algorithmic bytes of dispatch + combine divided by the step time.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per dispatch+combine and effective HBM GB/s (% of peak) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0


def algorithmic_bytes(sh, row_d: int, quant: bool) -> dict:
    """Bytes the method must move, per stage and per step.

    x read once, the send buffer written and read (the transfer is pulled by
    the receiver), the grouped layout written, the expert output read, the
    combined tokens written, plus the routing ids and weights. The
    quantising sender reads the bf16 rows (2H bytes) instead of fp8 ones.
    """
    N, T, R, H = sh.n_ranks, sh.tokens, sh.topk, sh.hidden
    NT, NTR, row_c = N * T, N * T * R, 2 * H
    row_x = 2 * H if quant else row_d
    stages = {
        "plan": 4 * NTR,                                  # routing ids
        "pack": NT * row_x + NTR * row_d,                 # read x, write send
        "recv": 2 * NTR * row_d,                          # read send, write grouped
        "combine": NTR * row_c + NT * row_c + 4 * NTR,    # read y and weights, write out
    }
    return {"stages": stages, "step": sum(stages.values())}


# Device sources each stage's kernels are built from (recorded counters of a
# kernel stay valid while these files are unchanged).
STAGE_SOURCES = {
    "plan": ["ep_plan.hip", "ep_plan_device.hpp", "ep_kernels.hpp", "ep_device.hpp"],
    "pack": ["ep_dispatch.hip", "ep_device.hpp"],
    "pack_quant": ["ep_quant.hip", "ep_device.hpp"],
    "recv": ["ep_dispatch.hip", "ep_device.hpp"],
    "combine": ["ep_combine.hip", "ep_device.hpp"],
    "plan_local": ["ep_plan.hip", "ep_plan_device.hpp", "ep_kernels.hpp", "ep_device.hpp"],
    "pack_exchange": ["ep_dispatch.hip", "ep_plan_device.hpp", "ep_kernels.hpp",
                      "ep_device.hpp"],
    "pack_quant_exchange": ["ep_quant.hip", "ep_plan_device.hpp", "ep_kernels.hpp",
                            "ep_device.hpp"],
}


def kernel_source_hash(files) -> str:
    """Hash of the code (comments and blank lines dropped) of the named device
    sources under combine_ep_plan_amd/csrc."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(ROOT, "combine_ep_plan_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, stage: str):
    """HBM bytes per launch of the stage's kernel from the committed
    rocprofv3 counter summary of this workload, or None if there is none or
    the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    k = rec.get("stages", {}).get(stage)
    if k is None or k.get("source_sha256_16") != kernel_source_hash(STAGE_SOURCES[stage]):
        return None
    return k["traffic_bytes"]


def cpu_baseline(sh, wl, budget_s: float, quant: bool) -> dict:
    """The oracle as it stands, single thread, on the same workload.

    With the quantising sender the oracle's quantiser (an exhaustive nearest
    code search per value) runs on the first `quant_ranks` source ranks only
    and its time is scaled by N / quant_ranks; the rest of the step runs on
    the whole workload.
    """
    import numpy as np
    import oracle

    N, T, E, R, H = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk, sh.hidden
    cap = oracle.recv_bound(N, T, E, R)
    quant_ranks = min(N, 2)
    times = []
    t_begin = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        p = oracle.plan(N, T, E, R, cap, wl.idx)
        totals = p["recv_off"][:, N]
        rows = int(min(cap, int(totals.max())))
        t_plan = time.perf_counter() - t0
        if quant:
            tq0 = time.perf_counter()
            oracle.dispatch_pack_quant(wl.x_bf16[:quant_ranks],
                                       {"send_pos": p["send_pos"][:quant_ranks]})
            t_pack = (time.perf_counter() - tq0) * N / quant_ranks
            # the full-size send planes from the pre-quantised rows (the same
            # bytes); this copy is not timed
            send = [oracle.dispatch_pack(pl, p) for pl in wl.planes]
        else:
            tp0 = time.perf_counter()
            send = [oracle.dispatch_pack(pl, p) for pl in wl.planes]
            t_pack = time.perf_counter() - tp0
        tr0 = time.perf_counter()
        recv = [oracle.transfer(s, p, rows) for s in send]
        grouped = [oracle.unpack(r, p, rows) for r in recv]
        t_recv = time.perf_counter() - tr0
        y = oracle.expert_op(grouped, p, H, sh.payload, wl.alpha)   # stand-in, not timed
        tc0 = time.perf_counter()
        out = oracle.combine(y, wl.weights, wl.idx, p)
        t_comb = time.perf_counter() - tc0
        times.append(t_plan + t_pack + t_recv + t_comb)
        del send, recv, grouped, y, out
        if time.perf_counter() - t_begin >= budget_s or len(times) >= 50:
            break
    return {"seconds": times, "median_s": statistics.median(times), "runs": len(times),
            "quant_ranks": quant_ranks if quant else None}


def measure_split(ep, torch, d, b, sh, P: int, steps: int, warmup: int) -> dict:
    """The split dispatch (sender half, receiver half with private regions of
    P rows) + combine, and its overlap with independent work: a stand-in for
    a shared expert (two bf16 GEMMs, H -> 2048 -> H, over all N*T tokens,
    random weights) on a second stream."""
    import statistics as st

    priv = ep.priv_buffers(d, P) if P > 0 else []
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()
    spa = sa.cuda_stream

    def send():
        ep.dispatch_send(d, b.idx, b.x, b.plan_ws, b.send, priv, P, b.status, spa)

    def recv():
        ep.dispatch_recv_split(d, b.send, priv, P, b.plan_ws, b.grouped, b.status, spa)

    def comb():
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, spa)

    NT, H = sh.n_ranks * sh.tokens, sh.hidden
    g = torch.Generator(device="cuda").manual_seed(1)
    xs = torch.randn(NT, H, device="cuda", dtype=torch.bfloat16, generator=g)
    w1 = torch.randn(H, 2048, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
    w2 = torch.randn(2048, H, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02

    def gemm():
        return torch.mm(torch.mm(xs, w1), w2)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = []
        for _ in range(reps):
            e0.record(sa)
            fn()
            e1.record(sa)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3)
        return st.median(out)

    def split_step():
        send()
        recv()
        comb()

    def split_overlapped():
        # the exchange on the second stream while the first one packs
        ep.dispatch_send_plan(d, b.idx, b.plan_ws, b.status, spa)
        counts = torch.cuda.Event()
        counts.record(sa)
        sb.wait_event(counts)
        ep.dispatch_recv_plan(d, b.plan_ws, b.status, sb.cuda_stream)
        offsets = torch.cuda.Event()
        offsets.record(sb)
        ep.dispatch_send_pack(d, b.idx, b.x, b.plan_ws, b.send, priv, P, spa)
        sa.wait_event(offsets)
        ep.dispatch_recv_pull(d, b.send, priv, P, b.plan_ws, b.grouped, spa)
        comb()

    def sequential():
        send()
        gemm()
        recv()
        comb()

    def overlapped():
        # the GEMM starts with the sender half on the second stream; the
        # step ends when both streams are done
        start = torch.cuda.Event()
        start.record(sa)
        sb.wait_event(start)
        with torch.cuda.stream(sb):
            gemm()
        split_step()
        done = torch.cuda.Event()
        done.record(sb)
        sa.wait_event(done)

    for fn in (split_step, split_overlapped, gemm, sequential, overlapped):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    stages = {"send": [], "recv": [], "combine": []}
    for _ in range(max(steps // 10, 3)):
        ev[0].record(sa)
        send()
        ev[1].record(sa)
        recv()
        ev[2].record(sa)
        comb()
        ev[3].record(sa)
        torch.cuda.synchronize()
        for j, n in enumerate(stages):
            stages[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(sa)
    for _ in range(steps):
        split_step()
    e1.record(sa)
    torch.cuda.synchronize()
    t_split = e0.elapsed_time(e1) / steps * 1e3
    e0.record(sa)
    for _ in range(steps):
        split_overlapped()
    e1.record(sa)
    torch.cuda.synchronize()
    t_ovl_step = e0.elapsed_time(e1) / steps * 1e3
    reps = max(steps // 5, 5)
    t_gemm = timed(gemm, reps)
    t_seq = timed(sequential, reps)
    t_ovl = timed(overlapped, reps)
    return {
        "priv_rows": P,
        "us_per_dispatch_combine": round(t_split, 2),
        "stages_us": {n: round(st.mean(v), 2) for n, v in stages.items()},
        "us_exchange_overlapped_with_pack": round(t_ovl_step, 2),
        "shared_expert_stand_in": f"bf16 GEMMs [{NT},{H}]x[{H},2048] then x[2048,{H}]",
        "shared_expert_us": round(t_gemm, 2),
        "sequential_us": round(t_seq, 2),
        "overlapped_us": round(t_ovl, 2),
    }


def measure_presum(ep, torch, np, d, b, sh, wl, steps: int, warmup: int) -> dict:
    """Combine with partial sums on the expert side next to the plain
    combine: time, and the rows a multi-GPU combine would move back (one per
    (token, rank) pair instead of one per slot)."""
    import statistics as st

    N, T, R, H, E = sh.n_ranks, sh.tokens, sh.topk, sh.hidden, sh.n_experts
    L = E // N
    ranks = wl.idx // L
    pairs = sum(len(set(row)) for row in ranks.reshape(-1, R).tolist())
    partial = torch.empty((N, T * R, H), dtype=torch.int16, device="cuda")
    out = torch.empty((N, T, H), dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream()
    sp = s.cuda_stream

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        res = []
        for _ in range(5):
            e0.record(s)
            for _ in range(max(steps // 5, 1)):
                fn()
            e1.record(s)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / max(steps // 5, 1) * 1e3)
        return st.median(res)

    t_plain = timed(lambda: ep.combine(d, b.expert_out, b.weights, b.plan_ws, out, sp))
    t_pre = timed(lambda: ep.combine_presum(d, b.expert_out, b.weights, b.plan_ws, partial,
                                            out, sp))
    row = 2 * H
    NT, NTR = N * T, N * T * R
    one_gpu = NTR * row + 2 * pairs * row + NT * row + 4 * NTR
    return {
        "combine_us": round(t_plain, 2),
        "presum_combine_us": round(t_pre, 2),
        "rows_returned": pairs,
        "rows_returned_plain": NTR,
        "returned_fraction": round(pairs / NTR, 4),
        "presum_bytes_one_gpu": one_gpu,
        "presum_GBps_one_gpu": round(one_gpu / t_pre / 1e3, 1),
    }


def measure_kv(ep, torch, np, W, reps: int = 10) -> dict:
    """KV-block push of one 16k-token request to 8 tensor-parallel ranks
    (Qwen3-32B shapes, 16-token blocks): merged regions, per-block
    descriptors, and the staged relay through 32 KiB x 64 bounce slots in
    device memory and in pinned host memory."""
    import statistics as st

    sh = W.KV_CONFIGS["kv_qwen32b_16k"]
    src_t, dst_t = W.make_kv_tables(sh)
    tok = sh.token_bytes
    bs, bd = sh.src_block_tokens, sh.dst_block_tokens
    src = torch.randint(0, 256, (sh.ranks, sh.src_pool_blocks * bs * tok), dtype=torch.uint8,
                        device="cuda")
    dst = torch.zeros((sh.ranks, sh.dst_pool_blocks * bd * tok), dtype=torch.uint8, device="cuda")
    notify = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    sp = s.cuda_stream
    total = sh.tokens * tok
    moved = 2 * total * sh.ranks            # read + write, all ranks
    res = {"workload": (f"{sh.name}: {sh.tokens} tokens x {tok} B per rank, {sh.ranks} ranks, "
                        f"{bs}-token blocks, free-list runs of mean {sh.src_mean_run:g} (source) "
                        f"and {sh.dst_mean_run:g} (destination) blocks"),
           "bytes_per_push": moved}
    bounce_dev = torch.empty(64 * 32768, dtype=torch.uint8, device="cuda")
    bounce_host = torch.empty(64 * 32768, dtype=torch.uint8, pin_memory=True)
    for name, merge, fn in (
            ("merged", True, lambda r, m: ep.kv_push(sh.ranks, r, m, total, src, src.shape[1],
                                                     dst, dst.shape[1], notify, status, sp)),
            ("per_block", False, lambda r, m: ep.kv_push(sh.ranks, r, m, total, src, src.shape[1],
                                                         dst, dst.shape[1], notify, status,
                                                         sp)),
            ("staged_device", True, lambda r, m: ep.kv_push_staged(
                sh.ranks, r, m, total, src, src.shape[1], dst, dst.shape[1], bounce_dev, 64,
                notify, status, sp)),
            ("staged_pinned_host", True, lambda r, m: ep.kv_push_staged(
                sh.ranks, r, m, total, src, src.shape[1], dst, dst.shape[1], bounce_host, 64,
                notify, status, sp))):
        reg = ep.kv_plan(sh.tokens, tok, bs, src_t, bd, dst_t, merge=merge)
        reg_dev = torch.from_numpy(reg).cuda()
        n = 2 if name == "staged_pinned_host" else reps
        fn(reg_dev, len(reg))
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn(reg_dev, len(reg))
            e1.record(s)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        t = st.median(ts)
        res[name] = {"regions": int(len(reg)), "us": round(t, 1),
                     "GBps": round(moved / t / 1e3, 1)}
    res["notify_ok"] = int(notify.item()) == sh.ranks * (3 * reps + 4 + 2) and int(status.item()) == 0
    return res


def measure_staged(ep, torch, d, sh, wl, steps: int, warmup: int) -> dict:
    """The dispatch with the network write materialised (ep_dispatch_transfer
    into receive buffers, then ep_dispatch_unpack) against the receiver with
    the transfer fused in (ep_dispatch_recv)."""
    import statistics as st

    b = ep.Buffers(d, device="cuda:0", staged=True)
    b.idx.copy_(torch.from_numpy(wl.idx))
    b.weights.copy_(torch.from_numpy(wl.weights))
    for q, plane in enumerate(wl.planes):
        b.x[q].copy_(torch.from_numpy(plane))
    s = torch.cuda.current_stream()
    sp = s.cuda_stream
    ep.plan(d, b.idx, b.plan_ws, b.status, sp)
    ep.dispatch_pack(d, b.x, b.plan_ws, b.send, sp)

    def staged():
        ep.dispatch_transfer(d, b.send, b.plan_ws, b.recv, sp)
        ep.dispatch_unpack(d, b.recv, b.plan_ws, b.grouped, sp)

    def fused():
        ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp)

    out = {}
    for name, fn in (("transfer_then_unpack_us", staged), ("fused_pull_us", fused)):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
    del b
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--sample-every", type=int, default=10,
                    help="record per-stage events on every n-th timed step")
    ap.add_argument("--prequantized", action="store_true",
                    help="fp8 payloads: send pre-quantised rows with the plain sender "
                         "instead of quantising bf16 rows in the sender")
    ap.add_argument("--flushed-steps", type=int, default=20,
                    help="extra steps, each after a 1 GiB fill and a 1 GiB read that evict the caches, "
                         "timed one by one (reported beside the main figure)")
    ap.add_argument("--split", type=int, default=-1, metavar="P",
                    help="also measure the split dispatch with P private rows per "
                         "(destination, source) pair, alone and overlapped with a "
                         "shared-expert stand-in on a second stream")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps as one HIP graph and replay it (removes "
                         "launch overhead; matters for launch-bound small workloads)")
    ap.add_argument("--staged", action="store_true",
                    help="also time the materialised network write + unpack against the "
                         "fused receiver")
    ap.add_argument("--presum", action="store_true",
                    help="also measure the combine with partial sums on the expert side")
    ap.add_argument("--kv", action="store_true",
                    help="also measure the KV-block push (merged, per-block, staged)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle CPU work for the baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the EP group's ranks are virtual ranks on one "
              f"MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import combine_ep_plan_amd as ep
    import ep_workloads as W

    torch.cuda.set_device(0)
    sh = W.CONFIGS[args.config]
    wl = W.make_workload(sh)
    d = ep.make_desc(sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk, sh.payload)
    b = ep.Buffers(d, device="cuda:0")
    b.idx.copy_(torch.from_numpy(wl.idx))
    b.weights.copy_(torch.from_numpy(wl.weights))
    for q, plane in enumerate(wl.planes):
        b.x[q].copy_(torch.from_numpy(plane))
    alpha = torch.from_numpy(wl.alpha).cuda() if wl.alpha is not None else None
    quant = sh.payload == W.PAYLOAD_FP8_B128 and not args.prequantized
    x_bf16 = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda() if quant else None
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    row_d = sum(ep.row_bytes(d, q) for q in range(ep.num_planes(d)))

    def pack():
        if quant:
            ep.dispatch_pack_quant(d, x_bf16, b.plan_ws, b.send, sp)
        else:
            ep.dispatch_pack(d, b.x, b.plan_ws, b.send, sp)

    # expert outputs once (outside timing)
    ep.plan(d, b.idx, b.plan_ws, b.status, sp)
    pack()
    ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sp)
    torch.cuda.synchronize()
    if int(b.status.item()) != 0:
        print(f"plan status {b.status.item()}", file=sys.stderr)
        return 1

    def staged_step(ev=None):
        """The four calls one by one, with an event between stages."""
        if ev is not None:
            ev[0].record(stream)
        ep.plan(d, b.idx, b.plan_ws, b.status, sp)
        if ev is not None:
            ev[1].record(stream)
        pack()
        if ev is not None:
            ev[2].record(stream)
        ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp)
        if ev is not None:
            ev[3].record(stream)
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp)
        if ev is not None:
            ev[4].record(stream)

    def fused_step(ev=None):
        """ep_dispatch / ep_dispatch_quant (plan + pack + receive, the count
        exchange folded into the sender launch) and ep_combine."""
        if ev is not None:
            ev[0].record(stream)
        if quant:
            ep.dispatch_quant(d, b.idx, x_bf16, b.plan_ws, b.send, b.grouped, b.status, sp)
        else:
            ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status, sp)
        if ev is not None:
            ev[1].record(stream)
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp)
        if ev is not None:
            ev[2].record(stream)

    # A step is the one-call dispatch and the combine.
    step = fused_step
    n_ev = 3
    for _ in range(args.warmup):
        step()
    # Events only on every `sample_every`-th step: an event record between
    # two kernels costs a few microseconds of GPU time.
    sampled = list(range(0, args.steps, args.sample_every))
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for i in sampled}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(events.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    steps_ms = [ev[0].elapsed_time(ev[-1]) for ev in events.values()]
    dispatch_call_us = statistics.mean(ev[0].elapsed_time(ev[1]) for ev in events.values()) * 1e3

    graph_step_us = None
    if args.graph:
        # The same K steps captured once as a HIP graph (timing events cannot
        # be recorded inside a capture, so none are) and replayed: one launch
        # for K steps, which removes the per-call launch cost.
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap_stream):
            cs = cap_stream.cuda_stream
            for _ in range(args.steps):
                if quant:
                    ep.dispatch_quant(d, b.idx, x_bf16, b.plan_ws, b.send, b.grouped, b.status, cs)
                else:
                    ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status, cs)
                ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, cs)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_step_us = g0.elapsed_time(g1) * 1e3 / args.steps
        del graph
    # Per-stage times (and the dominant kernel's) from the four separate
    # calls, after the timed region; the receiver kernel is the same launch
    # in both forms of the step.
    stage_names = ["plan", "pack", "recv", "combine"]
    per = {n: [] for n in stage_names}
    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
                for _ in range(max(len(sampled), 5))]
    for _ in range(3):
        staged_step()
    for ev in stage_ev:
        staged_step()
        staged_step(ev)
    torch.cuda.synchronize()
    for ev in stage_ev:
        for j, n in enumerate(stage_names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    ab = algorithmic_bytes(sh, row_d, quant)
    eff = ab["step"] / (ms_per_step * 1e-3) / 1e9

    # the dominant kernel: the stage with the largest algorithmic bytes
    dom = max(ab["stages"], key=lambda k: ab["stages"][k])
    # Its launch duration: 20 launches back to back between two events (one
    # event pair per launch would add the event overhead to each), after a
    # fresh plan and sender pass so that it reads what the sender wrote.
    dom_call = {"plan": lambda: ep.plan(d, b.idx, b.plan_ws, b.status, sp),
                "pack": pack,
                "recv": lambda: ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp),
                "combine": lambda: ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp)}[dom]
    ep.plan(d, b.idx, b.plan_ws, b.status, sp)
    pack()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(20):
        dom_call()
    k1.record(stream)
    torch.cuda.synchronize()
    dom_ms = k0.elapsed_time(k1) / 20
    achieved = ab["stages"][dom] / (dom_ms * 1e-3) / 1e9

    # the stand-in expert, outside the step (reported, not part of the metric)
    x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x0.record(stream)
    for _ in range(5):
        ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sp)
    x1.record(stream)
    torch.cuda.synchronize()
    expert_us = x0.elapsed_time(x1) / 5 * 1e3

    # copy ceiling of this GPU with the library's own row-copy loop (context)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        ep.probe_copy(dst, src, nbytes, sp)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        ep.probe_copy(dst, src, nbytes, sp)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9

    # Cold-cache steps: before each one (outside the events) a 1 GiB fill and
    # a 1 GiB read with ordinary stores and loads evict what the previous step
    # left in the L2s and the MALL. (The library's copy probe would not: its
    # non-temporal accesses leave cached lines in place, and so do the
    # receiver's and the combine's, which is why back-to-back steps find the
    # previous sender's token rows still in each XCD's L2.) Each step is timed
    # alone between two events.
    flushed = []
    for i in range(args.flushed_steps):
        dst.fill_(i & 0xff)
        src.view(torch.int32).max()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        step()
        f1.record(stream)
        torch.cuda.synchronize()
        flushed.append(f0.elapsed_time(f1) * 1e3)
    del src, dst

    split = None
    if args.split >= 0:
        split = measure_split(ep, torch, d, b, sh, args.split, args.steps, args.warmup)

    presum = None
    if args.presum:
        presum = measure_presum(ep, torch, np, d, b, sh, wl, args.steps, args.warmup)

    staged = None
    if args.staged:
        staged = measure_staged(ep, torch, d, sh, wl, max(args.steps // 5, 10), 3)

    kv = None
    if args.kv:
        kv = measure_kv(ep, torch, np, W)

    cpu = None
    if args.cpu_budget > 0:
        base = cpu_baseline(sh, wl, args.cpu_budget, quant)
        sample = (f"the whole {sh.name} workload, {base['runs']} run(s) of the plain-C "
                  f"oracle (plan, pack, per-pair transfer, unpack, combine; stand-in "
                  f"expert not timed), median {base['median_s']:.3f} s")
        if quant:
            sample += (f"; the quantising sender timed on {base['quant_ranks']} of "
                       f"{sh.n_ranks} source ranks and scaled")
        cpu = {
            "value": ab["step"] / base["median_s"] / 1e9,
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": sample,
            "us_per_step": base["median_s"] * 1e6,
        }

    if sh.payload == W.PAYLOAD_BF16:
        payload_name = "bf16"
    elif quant:
        payload_name = "fp8 e4m3 + fp32 scale per 128 values, quantised in the sender"
    else:
        payload_name = "fp8 e4m3 + fp32 scale per 128 values, pre-quantised"
    traffic = recorded_traffic(args.config, "pack_quant" if dom == "pack" and quant else dom)
    res = {
        "metric": METRIC,
        "value": round(eff, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{sh.name}: N={sh.n_ranks} virtual ranks, T={sh.tokens} tokens/rank, "
                         f"H={sh.hidden} bf16 tokens, dispatch payload {payload_name}, "
                         f"E={sh.n_experts} experts, top-{sh.topk} {sh.routing} routing, "
                         f"softmax weights, stand-in expert = {sh.expert}"),
            "parallelism": "ep (virtual ranks on one GPU)",
            "global_batch": sh.n_ranks * sh.tokens,
        },
        "us_per_dispatch_combine": round(ms_per_step * 1e3, 2),
        "us_per_virtual_rank": round(ms_per_step * 1e3 / sh.n_ranks, 3),
        "expert_stand_in_us": round(expert_us, 2),
        "frac_of_hbm_peak": round(eff / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": ab["step"],
        "step_form": ("ep_dispatch_quant" if quant else "ep_dispatch") +
                     " (plan + pack + recv) then ep_combine",
        "dispatch_call_us": round(dispatch_call_us, 2),
        **({"graph_step_us": round(graph_step_us, 2),
            "graph_from": "the K steps captured as one HIP graph, one replay between two events"}
           if graph_step_us is not None else {}),
        "stages_us": {n: round(statistics.mean(per[n]) * 1e3, 2) for n in stage_names},
        "stages_from": "the four separate calls, sampled after the timed steps",
        "instrumented_step_us_p10_p50_p90": [round(float(np.percentile(steps_ms, q)) * 1e3, 2)
                                             for q in (10, 50, 90)],
        "instrumented_steps": len(steps_ms),
        "cold_cache_step_us_p10_p50_p90": ([round(float(np.percentile(flushed, q)), 2)
                                            for q in (10, 50, 90)] if flushed else None),
        "wall_ms": round(wall_ms, 3),
        "roofline": {
            "kernel": f"ep_dispatch_{dom}" if dom in ("pack", "recv") else f"ep_{dom}",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_GBps": None if traffic is None else round(traffic / (dom_ms * 1e-3) / 1e9, 2),
            "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
            "algorithmic_bytes": ab["stages"][dom],
            "avg_us": round(dom_ms * 1e3, 2),
            "avg_us_from": "20 launches back to back between two HIP events on the launch stream",
        },
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "cpu_baseline": cpu,
    }
    if split is not None:
        res["split"] = split
    if presum is not None:
        res["presum"] = presum
    if kv is not None:
        res["kv_push"] = kv
    if staged is not None:
        res["staged_receive"] = staged
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

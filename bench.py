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


def cpu_host() -> dict:
    """Host CPU of this run: the model name, the logical CPUs the OS reports
    and the CPUs this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "cpus_allowed": affinity, "model": model}


def cpu_baseline(sh, wl, budget_s: float, quant: bool) -> dict:
    """The oracle as it stands, single thread, on the same workload.

    With the quantising sender the oracle's quantiser (an exhaustive nearest
    code search per value) runs on the first `quant_ranks` source ranks only
    and its time is scaled by N / quant_ranks; the rest of the step runs on
    the whole workload. The last run's plan and combined tokens are kept for
    the parity check of the benchmarked buffers.
    """
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
        del send, recv, grouped, y
        if time.perf_counter() - t_begin >= budget_s or len(times) >= 50:
            break
    return {"seconds": times, "median_s": statistics.median(times), "runs": len(times),
            "quant_ranks": quant_ranks if quant else None, "plan": p, "out": out}


class Flusher:
    """Evicts the L2s and the MALL between timed steps: a 1 GiB fill and a
    1 GiB read with ordinary stores and loads, outside the timed events. (The
    library's copy probe would not do: its non-temporal accesses leave cached
    lines in place, and so do the receiver's and the combine's, which is why
    back-to-back steps find the previous sender's token rows still in each
    XCD's L2.)"""

    def __init__(self, torch):
        self.a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        self.b = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")

    def __call__(self, i: int) -> None:
        self.a.fill_(i & 0xFF)
        self.b.max()


def time_flushed(torch, stream, step, n: int, flush) -> list:
    """n steps, each after a cache flush, each timed alone between two HIP
    events on the step's stream (synchronised on both sides); µs."""
    out = []
    for i in range(n):
        flush(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3)
    return out


def time_back_to_back(torch, stream, step, n: int) -> float:
    """n steps queued back to back between two HIP events; µs per step."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def pcts(np, v) -> list:
    return [round(float(np.percentile(v, q)), 2) for q in (10, 50, 90)]


def bench_parity(ep, torch, np, d, b, sh, wl, quant: bool, oracle_out=None,
                 n_tokens: int = 256, seed: int = 0) -> dict:
    """Parity of the benchmarked buffers with the oracle, after the timed
    steps:
      - every plan table the oracle computes (cnt, send_off, send_pos,
        recv_off, grp_off, grp_pos) and the status word, bit for bit;
      - every send row and every delivered grouped row equal to the token
        row the oracle's plan puts there (compared on the device);
      - with the quantising sender, the send rows of sampled tokens equal to
        the oracle's quantiser applied to their bf16 rows;
      - out: every token against the oracle's whole-path result when given
        (oracle_out), else sampled tokens against the oracle's per-token
        combine; for identity and dequantising stand-ins also every token
        against the closed form (weights summing to one give back the one
        expert value exactly);
      - combine bar: 8e-3 relative per element (the stand-in experts give
        each token terms of one sign).
    """
    import oracle
    import ep_workloads as W

    N, T, E, R, H = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk, sh.hidden
    L = E // N
    cap = ep.capacity(d)
    p = oracle.plan(N, T, E, R, cap, wl.idx)
    res = {}
    # plan tables
    v = ep.plan_views(d, b.plan_ws)
    base = b.plan_ws.data_ptr()
    ws = b.plan_ws.cpu().numpy()
    bad_tables = []
    for f in ("cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos"):
        off = getattr(v, f) - base
        got = ws[off:off + 4 * p[f].size].view(np.int32).reshape(p[f].shape)
        if not np.array_equal(got, p[f]):
            bad_tables.append(f)
    status = int(b.status.item())
    res["plan_tables"] = "bit-exact" if not bad_tables else "differ: " + ",".join(bad_tables)
    res["status"] = status
    # every send row and delivered grouped row, on the device
    NTR = N * T * R
    ss, tt, _ = np.unravel_index(np.arange(NTR), (N, T, R))
    dd = wl.idx.reshape(-1) // L
    sp, gp = p["send_pos"].reshape(-1), p["grp_pos"].reshape(-1)
    bad_send = bad_grp = n_send = n_grp = 0
    for q in range(len(b.x)):
        for lo in range(0, NTR, 16384):
            sl = slice(lo, min(lo + 16384, NTR))
            ok_s = sp[sl] >= 0
            ok_g = gp[sl] >= 0
            si = torch.from_numpy(ss[sl]).cuda()
            ti = torch.from_numpy(tt[sl]).cuda()
            want = b.x[q][si, ti]
            spi = torch.from_numpy(np.where(ok_s, sp[sl], 0).astype(np.int64)).cuda()
            gpi = torch.from_numpy(np.where(ok_g, gp[sl], 0).astype(np.int64)).cuda()
            di = torch.from_numpy(np.where(ok_g, dd[sl], 0).astype(np.int64)).cuda()
            ms = torch.from_numpy(ok_s).cuda()
            mg = torch.from_numpy(ok_g).cuda()
            row_bad_s = (b.send[q][si, spi] != want).any(dim=-1) & ms
            row_bad_g = (b.grouped[q][di, gpi] != want).any(dim=-1) & mg
            bad_send += int(row_bad_s.sum().item())
            bad_grp += int(row_bad_g.sum().item())
            n_send += int(ok_s.sum())
            n_grp += int(ok_g.sum())
    res["send_rows_checked"] = n_send // len(b.x)
    res["send_rows_bad"] = bad_send
    res["grouped_rows_checked"] = n_grp // len(b.x)
    res["grouped_rows_bad"] = bad_grp
    rng = np.random.default_rng(seed)
    if quant:
        toks = rng.choice(N * T, size=min(N * T, 64), replace=False)
        s_, t_ = np.unravel_index(toks, (N, T))
        oc, osc = oracle.quantize_b128(wl.x_bf16[s_, t_])
        k_ = rng.integers(0, R, size=len(toks))
        rows = p["send_pos"][s_, t_, k_]
        keep = rows >= 0
        si = torch.from_numpy(s_[keep].astype(np.int64)).cuda()
        ri = torch.from_numpy(rows[keep].astype(np.int64)).cuda()
        gc = b.send[0][si, ri].cpu().numpy()
        gs = b.send[1][si, ri].cpu().numpy().view(np.float32)
        res["quantised_rows_checked"] = int(keep.sum())
        res["quantised_rows_bad"] = int((gc != oc[keep]).any(-1).sum() +
                                        (gs.view(np.uint32) != osc[keep].view(np.uint32)).any(-1).sum())
    # combined tokens
    out = b.out.cpu().numpy().view(np.uint16)

    def close(g, o):
        gf = W.bf16_bits_to_f32(g).astype(np.float64)
        of = W.bf16_bits_to_f32(o).astype(np.float64)
        return np.abs(gf - of) <= 8e-3 * np.abs(of)

    if oracle_out is not None:
        ok = close(out, oracle_out)
        res["out_tokens_vs_oracle"] = N * T
        res["out_elements_off"] = int((~ok).sum())
    else:
        toks = rng.choice(N * T, size=min(N * T, n_tokens), replace=False)
        s_, t_ = np.unravel_index(toks, (N, T))
        off = 0
        for i in range(len(toks)):
            row = [pl[s_[i], t_[i]] for pl in wl.planes]
            ys = [oracle.expert_row(row, int(e), sh.payload, H, wl.alpha) if 0 <= e < E else None
                  for e in wl.idx[s_[i], t_[i]]]
            want = oracle.combine_token(wl.weights[s_[i], t_[i]], ys)
            off += int((~close(out[s_[i], t_[i]], want)).sum())
        res["out_tokens_vs_oracle"] = len(toks)
        res["out_elements_off"] = off
    if sh.expert in ("identity", "dequant") and status == 0:
        g = b.out
        if sh.expert == "identity":
            want = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda()
        else:
            codes = b.x[0].view(torch.float8_e4m3fn).to(torch.float32)
            scales = b.x[1].view(torch.float32).repeat_interleave(128, dim=-1)
            want = (codes * scales).to(torch.bfloat16).view(torch.int16)
        same = (g == want) | (((g & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))   # +0 == -0
        res["out_tokens_closed_form"] = N * T
        res["out_tokens_closed_form_bad"] = int((~same.all(dim=-1)).sum().item())
    res["pass"] = (not bad_tables and bad_send == 0 and bad_grp == 0
                   and res.get("quantised_rows_bad", 0) == 0 and res["out_elements_off"] == 0
                   and res.get("out_tokens_closed_form_bad", 0) == 0)
    return res


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


def measure_presum(ep, torch, np, d, b, sh, wl, alpha, steps: int, warmup: int) -> dict:
    """Combine with partial sums on the expert side next to the plain
    combine: time, the rows a multi-GPU combine would move back (one per
    (token, rank) pair instead of one per slot), and how far the partial
    sums' extra roundings move the result (every element, against the plain
    combine, relative to sum_k |w_k y_k|)."""
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
    # Accuracy: the partial-sum combine against the plain one, per element,
    # relative to sum_k |w_k y_k| (the plain combine of |y| with |w|: the
    # library computes the denominators too). The plain combine itself is
    # within the parity bar of the exact sum.
    def f32(t):
        return (t.to(torch.int32) << 16).view(torch.float32)

    ep.combine(d, b.expert_out, b.weights, b.plan_ws, out, sp)
    plain = f32(out)
    ep.combine_presum(d, b.expert_out, b.weights, b.plan_ws, partial, out, sp)
    pre = f32(out)
    # |y| in place (the expert rows can be ~100 GB at prefill, no room for a
    # copy), then the stand-in expert writes them back as they were.
    b.expert_out.bitwise_and_(0x7FFF)
    ep.combine(d, b.expert_out, b.weights.abs(), b.plan_ws, out, sp)
    den = f32(out)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sp)
    torch.cuda.synchronize()
    live = den > 0
    rel = ((pre - plain).abs() / den.clamp_min(1e-30))[live]
    row = 2 * H
    NT, NTR = N * T, N * T * R
    one_gpu = NTR * row + 2 * pairs * row + NT * row + 4 * NTR
    return {
        "combine_us": round(t_plain, 2),
        "presum_combine_us": round(t_pre, 2),
        "presum_vs_plain_max_rel_to_sum_abs": float(rel.max().item()) if rel.numel() else 0.0,
        "presum_vs_plain_mean_rel_to_sum_abs": float(rel.mean().item()) if rel.numel() else 0.0,
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


def measure_probe(ep, torch, np, W, names, flush) -> dict:
    """Kernel-level probe behind the design's sender and copy figures (and
    the counter summaries under profiles/, which run it under rocprofv3):
      - per workload, steps of the four separate calls (ep_plan, the sender
        -- ep_dispatch_pack, or the quantising sender for fp8 workloads --,
        ep_dispatch_recv, ep_combine) with an event between stages: 3
        untimed, then 5 back to back, 5 each after a cache flush, and 5 each
        after a cache flush followed by a read of the token rows (torch max,
        ordinary loads); the median per stage (us);
      - the library's copy probe on 0.5, 1, 2 and 3 GiB, 3 launches each,
        each launch alone between two HIP events."""
    import gc

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    res = {}
    stage_names = ("plan", "sender", "recv", "combine")
    for name in names:
        sh, wl, d, b, alpha = setup(ep, torch, np, W, name)
        quant = sh.payload == W.PAYLOAD_FP8_B128
        xq = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda() if quant else None
        xs = xq if quant else b.x[0]

        def step(ev=None):
            calls = (lambda: ep.plan(d, b.idx, b.plan_ws, b.status, sp),
                     (lambda: ep.dispatch_pack_quant(d, xq, b.plan_ws, b.send, sp)) if quant
                     else (lambda: ep.dispatch_pack(d, b.x, b.plan_ws, b.send, sp)),
                     lambda: ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp),
                     lambda: ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp))
            for j, c in enumerate(calls):
                if ev is not None:
                    ev[j].record(stream)
                c()
            if ev is not None:
                ev[4].record(stream)

        def phase(pre):
            per = []
            for i in range(5):
                if pre is not None:
                    pre(i)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                step(ev)
                if pre is not None:
                    torch.cuda.synchronize()
                per.append(ev)
            torch.cuda.synchronize()
            return {n: round(float(np.median([e[j].elapsed_time(e[j + 1]) * 1e3 for e in per])), 2)
                    for j, n in enumerate(stage_names)}

        b.status.zero_()
        step()
        ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sp)
        step()
        step()
        torch.cuda.synchronize()
        row_d = sum(ep.row_bytes(d, q) for q in range(ep.num_planes(d)))
        res[name] = {
            "sender": "ep_dispatch_pack_quant" if quant else "ep_dispatch_pack",
            "algorithmic_bytes": algorithmic_bytes(sh, row_d, quant)["stages"],
            "back_to_back_us": phase(None),
            "after_flush_us": phase(flush),
            "after_flush_and_token_read_us": phase(
                lambda i: (flush(i), xs.view(torch.int32).max())),
        }
        del b, xq, xs
        gc.collect()
        torch.cuda.empty_cache()
    copies = {}
    for gib in (0.5, 1, 2, 3):
        n = int(gib * (1 << 30))
        src = torch.zeros(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ep.probe_copy(dst, src, n, sp)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(round(e0.elapsed_time(e1) * 1e3, 2))
        copies[f"{gib:g}GiB"] = {"us": ts, "TBps": [round(2 * n / t / 1e6, 3) for t in ts]}
        del src, dst
        torch.cuda.empty_cache()
    res["copy_probe"] = copies
    return res


def measure_sender_probe(ep, torch, np, W, flush) -> dict:
    """What limits the quantising sender on the prefill workload, through the
    public calls only (the figures of the design's sender section):
      - the fused sender (ep_dispatch_pack_quant) on the whole workload;
      - quantise once: the same call on a descriptor with one row per token
        whose ids all name expert 0, so that its send buffer is the quantised
        token rows in token order (a staging area);
      - the plain sender (ep_dispatch_pack, send order over windows for this
        descriptor) from pre-quantised rows: the generator's planes, back to
        back (their rows in the memory-side cache) and after a flush, and the
        staging rows right after the staging call wrote them;
      - one source sent alone (a descriptor with N = 1 and that source's
        ids): back to back, after a flush, and after a flush followed by a
        read of its token rows;
      - that source with 1, 2 or 4 rows per token (E = 32 R experts, uniform
        distinct ids drawn from a fixed seed): the time of the token reads and
        the quantisation against that of the extra rows;
      - the same loads and code-row stores with no arithmetic and no scale
        rows (the access-pattern probe's wide scatter at the plan's send
        positions), 1 or 7 KB of codes per wave, cached or non-temporal
        loads, back to back and after a flush.
    Each figure is the median of 5 launches, each timed alone between two
    HIP events. The byte-equality checks compare the two-pass and
    per-source send buffers with the fused sender's."""
    import gc

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    sh = W.CONFIGS["prefill"]
    wl = W.make_workload(sh)
    N, T, H, E, R = sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk
    F8 = ep.EP_PAYLOAD_FP8_B128
    u8 = torch.uint8
    d = ep.make_desc(N, T, H, E, R, F8)
    rows = [ep.row_bytes(d, q) for q in range(2)]
    idx = torch.from_numpy(wl.idx).cuda()
    x = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda()
    xq = [torch.from_numpy(pl).cuda() for pl in wl.planes]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = torch.empty(ep.plan_bytes(d), dtype=u8, device="cuda")
    send = [torch.empty((N, T * R, r), dtype=u8, device="cuda") for r in rows]
    ep.plan(d, idx, plan, status, sp)
    ds = ep.make_desc(N, T, H, N, 1, F8)
    plan_s = torch.empty(ep.plan_bytes(ds), dtype=u8, device="cuda")
    ep.plan(ds, torch.zeros((N, T, 1), dtype=torch.int32, device="cuda"), plan_s, status, sp)
    stg = [torch.empty((N, T, r), dtype=u8, device="cuda") for r in rows]

    def timed(fns, pre=None, reps=5):
        out = [[] for _ in fns]
        for i in range(reps):
            if pre is not None:
                pre(i)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            torch.cuda.synchronize()
            ev[0].record(stream)
            for j, fn in enumerate(fns):
                fn()
                ev[j + 1].record(stream)
            torch.cuda.synchronize()
            for j in range(len(fns)):
                out[j].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
        return [round(float(np.median(o)), 1) for o in out]

    fused = lambda: ep.dispatch_pack_quant(d, x, plan, send, sp)
    stage = lambda: ep.dispatch_pack_quant(ds, x, plan_s, stg, sp)
    copy_stg = lambda: ep.dispatch_pack(d, stg, plan, send, sp)
    copy_gen = lambda: ep.dispatch_pack(d, xq, plan, send, sp)
    fused()
    torch.cuda.synchronize()
    ref = [t.clone() for t in send]
    for t in send:
        t.zero_()
    stage()
    copy_stg()
    torch.cuda.synchronize()
    res = {"workload": describe(sh, W, True), "status": int(status.item()),
           "windowed_plain_sender": bool(ep.plan_views(d, plan).win_list),
           "staging_equals_generator_planes": all(torch.equal(a, c) for a, c in zip(stg, xq)),
           "two_pass_send_equals_fused": all(torch.equal(a, c) for a, c in zip(send, ref))}
    res["fused_us"] = {"back_to_back": timed([fused, fused])[1], "after_flush": timed([fused], flush)[0]}
    res["staging_pass_us"] = {"back_to_back": timed([stage, stage])[1],
                              "after_flush": timed([stage], flush)[0]}
    res["plain_sender_us"] = {
        "generator_planes_back_to_back": timed([copy_gen, copy_gen])[1],
        "generator_planes_after_flush": timed([copy_gen], flush)[0],
        "staging_rows_right_after_the_staging_call": timed([stage, copy_stg])[1],
        "staging_rows_after_flush": timed([copy_stg], flush)[0]}
    del stg, plan_s
    gc.collect()
    # one source alone
    d1 = ep.make_desc(1, T, H, E, R, F8)
    plan1 = torch.empty(ep.plan_bytes(d1), dtype=u8, device="cuda")
    ep.plan(d1, idx[0:1].contiguous(), plan1, status, sp)
    x0 = x[0:1]
    send1 = [t[0:1] for t in send]
    one = lambda: ep.dispatch_pack_quant(d1, x0, plan1, send1, sp)
    for t in send:
        t.zero_()
    one()
    torch.cuda.synchronize()
    res["one_source_send_equals_fused"] = all(torch.equal(a[0], c[0]) for a, c in zip(send, ref))
    res["one_source_us"] = {
        "back_to_back": timed([one, one])[1],
        "after_flush": timed([one], flush)[0],
        "after_flush_and_token_read": timed([lambda: x0.view(torch.int32).max(), one], flush)[1]}
    rng = np.random.default_rng(7)
    rsweep = {}
    for r in (1, 2, 4, R):
        e_r = 32 * r
        dr = ep.make_desc(1, T, H, e_r, r, F8)
        ids = np.argsort(rng.random((1, T, e_r)), axis=-1, kind="stable")[..., :r].astype(np.int32)
        plan_r = torch.empty(ep.plan_bytes(dr), dtype=u8, device="cuda")
        ep.plan(dr, torch.from_numpy(ids).cuda(), plan_r, status, sp)
        send_r = [torch.empty((1, T * r, ep.row_bytes(dr, q)), dtype=u8, device="cuda") for q in range(2)]
        fn = lambda: ep.dispatch_pack_quant(dr, x0, plan_r, send_r, sp)
        fn()
        rsweep[f"R={r},E={e_r}"] = {"back_to_back": timed([fn, fn])[1]}
        del send_r, plan_r
    res["one_source_rows_per_token_us"] = rsweep
    # The fused sender's loads and code-row stores without its arithmetic and
    # scale rows: each bf16 token row read once, narrowed 2:1 (xor of
    # adjacent 16-byte chunks) and written to its R send rows at the plan's
    # stable positions, in token order (the access-pattern probe's wide
    # scatter). It overwrites the code plane, so it runs last.
    order = np.argsort(wl.idx.reshape(N, T * R), axis=1, kind="stable")
    pos = np.empty_like(order)
    np.put_along_axis(pos, order, np.arange(T * R)[None, :], axis=1)
    table = torch.from_numpy(
        (np.arange(N)[:, None] * T * R + pos).astype(np.int32).reshape(-1)).cuda()
    codes = send[0].view(N * T * R, rows[0])
    bare = {}
    for kb in (1, 7):
        for name, fl in (("cached", 0), ("nt", ep.EP_PROBE_NT_LOADS)):
            fn = lambda: ep.probe_pattern(codes, x, table, N * T, N * T * R, rows[0], kb * 1024,
                                          fan_in=R, mode=ep.EP_PROBE_SCATTER_WIDE, flags=fl,
                                          stream=sp)
            bare[f"{kb}KB_per_wave_{name}_loads"] = {"back_to_back": timed([fn, fn])[1],
                                                     "after_flush": timed([fn], flush)[0]}
    res["bare_scatter_bytes"] = N * T * 2 * H + N * T * R * rows[0]
    res["bare_scatter_us"] = bare
    torch.cuda.synchronize()
    res["status_after"] = int(status.item())
    return res


def measure_pattern_probe(ep, torch, np, W, flush, reps: int = 5) -> dict:
    """The access shapes the sender, receiver and combine were chosen on,
    through the library's access-pattern probe (ep_probe_pattern). Each
    figure is the median of `reps` launches, each alone between two HIP
    events (back to back unless stated):
      - fills of 1 GiB: one piece of 1, 4, 14 or 64 KB per wave in output
        order, and 1 KB pieces walked grid-stride by 2048 or 8192 waves;
      - copies of 1 GiB: 1 KB per wave, the library's copy probe (7 KB per
        wave) and torch's device-to-device copy;
      - copies of the decode size (32768 rows of 14 KB, 470 MB out): linear,
        rows permuted at random, and sender-like (each of the 4096 token rows
        read 8 times, in the send order of the decode routing: per source,
        slots stably sorted by expert) with cached loads and the XCD
        renumbering, without the renumbering, and with non-temporal loads;
        1, 2, 7 and 14 KB per wave;
      - the receiver's row pairs at the decode size in receive order (the
        library's) and in send order (a scatter);
      - workgroups of four waves against one wave at the decode size, 1 KB
        per wave: linear copy, rows permuted, the receiver's pairs in
        receive order, the combine's mix (8 rows in flight), fill and read;
      - the combine's mix: 4096 rows of 14 KB, each the xor of 8 rows from 8
        linear regions (470 MB read, 59 MB written), 1, 2, 7 and 14 KB per
        wave, 2 or 8 rows in flight, cached and non-temporal loads; the same
        470 MB read only;
      - memory-side cache reuse: 32, 128 and 512 MB read (non-temporal and
        cached loads) right after a fill of the same bytes, right after a
        read of them, and after a flush;
      - the sender's two orders by bytes per source: 8 sources of 128 to
        2048 token rows of 14 KB (1.8 to 29 MB each), top-8 of 256 experts,
        uniform routing; send order (the gather above: cached loads, XCD
        renumbering, 1 KB per wave) against token order (a scatter: each
        token row read once, non-temporal loads, and written to its 8 send
        rows, 1 KB or 14 KB per wave)."""
    import gc

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    COPY, FILL, READ = ep.EP_PROBE_COPY, ep.EP_PROBE_FILL, ep.EP_PROBE_READ
    NTL, XCD = ep.EP_PROBE_NT_LOADS, ep.EP_PROBE_XCD

    def probe(dst, src, table, rows, src_rows, row, piece, **kw):
        return lambda: ep.probe_pattern(dst, src, table, rows, src_rows, row, piece,
                                        stream=sp, **kw)

    def timed(fn, pre=None):
        ts = []
        for i in range(reps):
            if pre is not None:
                pre(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    def fig(fn, nbytes, pre=None):
        us = timed(fn, pre)
        return {"us": round(us, 2), "TBps": round(nbytes / us / 1e6, 3)}

    res = {}
    # Fills of 1 GiB.
    GiB = 1 << 30
    a = torch.empty(GiB + (1 << 20), dtype=torch.uint8, device="cuda")
    fills = {}
    for kb in (1, 4, 14, 64):
        row = 14336 if kb == 14 else 65536
        rows = GiB // row
        fills[f"{kb}KB_per_wave"] = fig(probe(a, None, None, rows, 0, row, kb * 1024, mode=FILL),
                                        rows * row)
    for waves in (2048, 8192):
        fills[f"1KB_grid_stride_{waves}_waves"] = fig(
            probe(a, None, None, GiB // 65536, 0, 65536, 1024, mode=FILL, waves=waves), GiB)
    res["fill_1GiB"] = fills
    # Copies of 1 GiB (bytes read + written): the pattern probe's linear copy,
    # the library's copy probe (7 KB per wave) and torch's device copy.
    b = torch.empty_like(a)
    rows = GiB // 65536
    res["copy_1GiB"] = {
        "1KB_per_wave_nt_loads": fig(probe(b, a, None, rows, rows, 65536, 1024, flags=NTL),
                                     2 * GiB),
        "ep_probe_copy_7KB_per_wave": fig(lambda: ep.probe_copy(b, a, GiB, sp), 2 * GiB),
        "torch_copy_": fig(lambda: b[:GiB].copy_(a[:GiB]), 2 * GiB),
    }
    del a, b
    torch.cuda.empty_cache()

    # Copies at the decode size.
    sh = W.CONFIGS["decode"]
    N, T, R, row = sh.n_ranks, sh.tokens, sh.topk, 2 * sh.hidden
    rng = np.random.default_rng(sh.seed)
    idx = W.make_workload(sh).idx.reshape(N, T * R)
    order = np.argsort(idx, axis=1, kind="stable")           # send row -> slot, per source
    send_table = (np.arange(N)[:, None] * T + order // R).astype(np.int32).reshape(-1)
    nrows = N * T * R
    src_big = torch.randint(0, 255, (nrows, row), dtype=torch.uint8, device="cuda")
    src_tok = src_big[:N * T]
    dst = torch.empty_like(src_big)
    perm = torch.from_numpy(rng.permutation(nrows).astype(np.int32)).cuda()
    sendt = torch.from_numpy(send_table).cuda()
    copy_bytes = 2 * nrows * row
    send_bytes = N * T * row + nrows * row
    copies = {}
    for kb in (1, 2, 7, 14):
        pb = kb * 1024
        copies[f"{kb}KB_per_wave"] = {
            "linear": fig(probe(dst, src_big, None, nrows, nrows, row, pb, flags=NTL),
                          copy_bytes),
            "rows_permuted": fig(probe(dst, src_big, perm, nrows, nrows, row, pb, flags=NTL),
                                 copy_bytes),
            "sender_like_cached_xcd": fig(
                probe(dst, src_tok, sendt, nrows, N * T, row, pb, flags=XCD), send_bytes),
            "sender_like_cached": fig(probe(dst, src_tok, sendt, nrows, N * T, row, pb),
                                      send_bytes),
            "sender_like_nt_xcd": fig(
                probe(dst, src_tok, sendt, nrows, N * T, row, pb, flags=NTL | XCD), send_bytes),
        }
    res["copy_decode_size"] = {
        "bytes": {"linear_and_permuted": copy_bytes, "sender_like": send_bytes},
        "figures": copies}

    # The receiver's row pairs (send row -> grouped row of the decode
    # routing) in two orders, 1 KB per wave, non-temporal loads: receive
    # order (grouped rows written in order, send rows read as the table
    # says) and send order (send rows read in order, grouped rows written
    # where they belong: a scatter of one row each).
    TR = T * R
    pos = np.empty_like(order)
    np.put_along_axis(pos, order, np.arange(TR)[None, :], axis=1)
    send_row = (np.arange(N)[:, None] * TR + pos).reshape(-1)    # slot -> send row
    recv_order = np.argsort(idx.reshape(-1), kind="stable")      # grouped row -> slot
    grouped_of_slot = np.empty(nrows, np.int64)
    grouped_of_slot[recv_order] = np.arange(nrows)
    slot_of_send_row = (np.arange(N)[:, None] * TR + order).reshape(-1)
    gather_t = torch.from_numpy(send_row[recv_order].astype(np.int32)).cuda()
    scatter_t = torch.from_numpy(grouped_of_slot[slot_of_send_row].astype(np.int32)).cuda()
    res["receiver_orders_decode_size"] = {
        "bytes": copy_bytes,
        "receive_order": fig(probe(dst, src_big, gather_t, nrows, nrows, row, 1024, flags=NTL),
                             copy_bytes),
        "send_order": fig(probe(dst, src_big, scatter_t, nrows, nrows, row, 1024,
                                mode=ep.EP_PROBE_SCATTER, flags=NTL), copy_bytes),
    }

    # Workgroup size: the same shapes with workgroups of four waves (the
    # library's default) and of one wave (the receiver's), 1 KB per wave,
    # non-temporal loads.
    out_rows = N * T
    wg = {}
    for name, fl in (("four_waves", NTL), ("one_wave", NTL | ep.EP_PROBE_ONE_WAVE)):
        wg[name] = {
            "linear_copy": fig(probe(dst, src_big, None, nrows, nrows, row, 1024, flags=fl),
                               copy_bytes),
            "rows_permuted": fig(probe(dst, src_big, perm, nrows, nrows, row, 1024, flags=fl),
                                 copy_bytes),
            "receiver_pairs_receive_order": fig(
                probe(dst, src_big, gather_t, nrows, nrows, row, 1024, flags=fl), copy_bytes),
            "combine_mix_8_in_flight": fig(
                probe(dst[:out_rows], src_big, None, out_rows, nrows, row, 1024, fan_in=8,
                      in_flight=8, flags=fl), nrows * row + out_rows * row),
            "fill": fig(probe(dst, None, None, nrows, 0, row, 1024, mode=FILL,
                              flags=fl & ep.EP_PROBE_ONE_WAVE), nrows * row),
            "read": fig(probe(dst[:1], src_big, None, nrows, nrows, row, 1024, mode=READ,
                              flags=fl), nrows * row),
        }
    res["workgroup_size_decode_size"] = wg
    del gather_t, scatter_t

    # The combine's 8:1 mix over the same 470 MB.
    out_rows = N * T
    out = dst[:out_rows]
    mix_bytes = nrows * row + out_rows * row
    mix = {}
    for kb, inflight in ((1, 8), (2, 8), (7, 2), (14, 2), (14, 8)):
        for name, fl in (("cached", 0), ("nt", NTL)):
            mix[f"{kb}KB_per_wave_{inflight}_in_flight_{name}"] = fig(
                probe(out, src_big, None, out_rows, nrows, row, kb * 1024, fan_in=8,
                      in_flight=inflight, flags=fl), mix_bytes)
    for name, fl in (("cached", 0), ("nt", NTL)):
        mix[f"read_only_1KB_{name}"] = fig(
            probe(out, src_big, None, nrows, nrows, row, 1024, mode=READ, flags=fl),
            nrows * row)
    res["combine_mix_decode_size"] = {"bytes": mix_bytes, "figures": mix}
    del src_big, src_tok, dst, out, perm, sendt
    gc.collect()
    torch.cuda.empty_cache()

    # Reuse from the memory-side cache.
    reuse = {}
    for mb in (32, 128, 512):
        n = mb << 20
        buf = torch.empty(n, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        rows = n // 65536
        fill = probe(buf, None, None, rows, 0, 65536, 1024, mode=FILL)
        entry = {}
        for name, fl in (("nt", NTL), ("cached", 0)):
            rd = probe(sink, buf, None, rows, rows, 65536, 1024, mode=READ, flags=fl)
            entry[f"{name}_after_fill"] = fig(rd, n, pre=lambda i: fill())
            entry[f"{name}_after_read"] = fig(rd, n, pre=lambda i: (flush(i), rd()))
            entry[f"{name}_after_flush"] = fig(rd, n, pre=lambda i: (fill(), flush(i)))
        reuse[f"{mb}MB"] = entry
        del buf, sink
        torch.cuda.empty_cache()
    res["mall_reuse"] = reuse

    # Send order against token order by bytes per source.
    SCATTER = ep.EP_PROBE_SCATTER
    orders = {}
    N, R, E = 8, 8, 256
    for T in (128, 256, 512, 1024, 2048):
        rng = np.random.default_rng(1000 + T)
        idx = np.argsort(rng.random((N, T, E)), axis=-1, kind="stable")[..., :R]
        order = np.argsort(idx.reshape(N, T * R), axis=1, kind="stable")
        gather = (np.arange(N)[:, None] * T + order // R).astype(np.int32).reshape(-1)
        pos = np.empty_like(order)
        np.put_along_axis(pos, order, np.arange(T * R)[None, :], axis=1)
        scatter = (np.arange(N)[:, None] * T * R + pos).astype(np.int32).reshape(-1)
        src = torch.randint(0, 255, (N * T, row), dtype=torch.uint8, device="cuda")
        dst = torch.empty((N * T * R, row), dtype=torch.uint8, device="cuda")
        gt = torch.from_numpy(gather).cuda()
        st = torch.from_numpy(scatter).cuda()
        nb = N * T * row + N * T * R * row
        orders[f"{T * row / 1e6:.1f}MB_per_source"] = {
            "tokens": T,
            "send_order_1KB": fig(probe(dst, src, gt, N * T * R, N * T, row, 1024, flags=XCD),
                                  nb),
            "token_order_1KB": fig(probe(dst, src, st, N * T, N * T * R, row, 1024, fan_in=R,
                                         mode=SCATTER, flags=NTL), nb),
            "token_order_14KB": fig(probe(dst, src, st, N * T, N * T * R, row, row, fan_in=R,
                                          mode=SCATTER, flags=NTL), nb),
        }
        del src, dst, gt, st
        torch.cuda.empty_cache()
    res["sender_orders_by_source_size"] = orders
    return res


def setup(ep, torch, np, W, name: str):
    """Workload, caller-owned buffers, inputs in HBM and the stand-in
    expert's output (computed once, outside any timing)."""
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    d = ep.make_desc(sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk, sh.payload)
    b = ep.Buffers(d, device="cuda:0")
    b.idx.copy_(torch.from_numpy(wl.idx))
    b.weights.copy_(torch.from_numpy(wl.weights))
    for q, plane in enumerate(wl.planes):
        b.x[q].copy_(torch.from_numpy(plane))
    alpha = torch.from_numpy(wl.alpha).cuda() if wl.alpha is not None else None
    return sh, wl, d, b, alpha


def describe(sh, W, quant: bool) -> str:
    if sh.payload == W.PAYLOAD_BF16:
        payload = "bf16"
    elif quant:
        payload = "fp8 e4m3 + fp32 scale per 128 values, quantised in the sender"
    else:
        payload = "fp8 e4m3 + fp32 scale per 128 values, pre-quantised"
    return (f"{sh.name}: N={sh.n_ranks} virtual ranks, T={sh.tokens} tokens/rank, "
            f"H={sh.hidden} bf16 tokens, dispatch payload {payload}, E={sh.n_experts} experts, "
            f"top-{sh.topk} {sh.routing} routing, softmax weights, stand-in expert = {sh.expert}")


# Per-config protocol: iterations, and whether a cache flush precedes each
# step (the large workloads) or the steps run back to back (the tiny ones,
# which are launch-bound and report microseconds only).
CONFIG_PROTOCOL = {"tiny": (200, False), "tiny_zipf": (200, False), "decode": (100, True),
                   "worst": (100, True), "prefill": (30, True), "decode_zipf": (100, True),
                   "decode_fp8": (100, True)}


def dominant_roofline(ep, torch, d, b, sh, quant, x_bf16, ab, workload, stream) -> dict:
    """The roofline object of a workload's dominant kernel (the stage with
    the largest algorithmic bytes): its launch duration over 20 launches
    back to back between two events (one event pair per launch would add
    the event overhead to each), after a fresh plan and sender pass so that
    it reads what the sender wrote; the counter traffic recorded for it
    under profiles/ while its sources hash the same."""
    sp = stream.cuda_stream
    dom = max(ab["stages"], key=lambda k: ab["stages"][k])

    def pack():
        if quant:
            ep.dispatch_pack_quant(d, x_bf16, b.plan_ws, b.send, sp)
        else:
            ep.dispatch_pack(d, b.x, b.plan_ws, b.send, sp)

    call = {"plan": lambda: ep.plan(d, b.idx, b.plan_ws, b.status, sp),
            "pack": pack,
            "recv": lambda: ep.dispatch_recv(d, b.send, b.plan_ws, b.grouped, sp),
            "combine": lambda: ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp)}[dom]
    ep.plan(d, b.idx, b.plan_ws, b.status, sp)
    pack()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(20):
        call()
    k1.record(stream)
    torch.cuda.synchronize()
    dom_ms = k0.elapsed_time(k1) / 20
    achieved = ab["stages"][dom] / (dom_ms * 1e-3) / 1e9
    traffic = recorded_traffic(workload, "pack_quant" if dom == "pack" and quant else dom)
    return {
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
    }


def run_config(ep, torch, np, W, name: str, flush, warmup: int = 20) -> dict:
    """One workload under its protocol: dispatch + combine steps timed on
    the device, then the parity of its buffers with the oracle (the whole
    oracle path for the tiny workloads, sampled tokens plus closed forms for
    the others)."""
    import oracle

    steps, flushed = CONFIG_PROTOCOL[name]
    sh, wl, d, b, alpha = setup(ep, torch, np, W, name)
    quant = sh.payload == W.PAYLOAD_FP8_B128
    x_bf16 = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda() if quant else None
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        if quant:
            ep.dispatch_quant(d, b.idx, x_bf16, b.plan_ws, b.send, b.grouped, b.status, sp)
        else:
            ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status, sp)
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out, sp)

    b.status.zero_()
    step()
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out, sp)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    row_d = sum(ep.row_bytes(d, q) for q in range(ep.num_planes(d)))
    ab = algorithmic_bytes(sh, row_d, quant)
    res = {"workload": describe(sh, W, quant), "steps": steps, "warmup": warmup,
           "step_form": ("ep_dispatch_quant" if quant else "ep_dispatch") + " then ep_combine",
           "algorithmic_bytes_per_step": ab["step"]}
    b2b = time_back_to_back(torch, stream, step, steps)
    if flushed:
        ts = time_flushed(torch, stream, step, steps, flush)
        us = statistics.median(ts)
        res.update(flushed=True, us_p10_p50_p90=pcts(np, ts),
                   us_mean=round(statistics.mean(ts), 2), back_to_back_us=round(b2b, 2))
    else:
        us = b2b
        res.update(flushed=False, us_back_to_back=round(b2b, 2))
    res["effective_GBps"] = round(ab["step"] / us / 1e3, 1)
    res["frac_of_hbm_peak"] = round(ab["step"] / us / 1e3 / HBM_PEAK_GBPS, 4)
    if flushed:
        res["roofline"] = dominant_roofline(ep, torch, d, b, sh, quant, x_bf16, ab, name, stream)
    if name in ("tiny", "tiny_zipf"):
        ref = oracle.run(wl, cap=ep.capacity(d))
        res["parity"] = bench_parity(ep, torch, np, d, b, sh, wl, quant, oracle_out=ref["out"])
    else:
        res["parity"] = bench_parity(ep, torch, np, d, b, sh, wl, quant)
    del b, x_bf16
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed steps of the headline workload, each after a cache flush")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--configs", default="tiny,tiny_zipf,prefill,worst",
                    help="further workloads measured under their own protocol and reported "
                         "in the line's 'configs' object ('' for none)")
    ap.add_argument("--sample-every", type=int, default=10,
                    help="record per-stage events on every n-th back-to-back step")
    ap.add_argument("--prequantized", action="store_true",
                    help="fp8 payloads: send pre-quantised rows with the plain sender "
                         "instead of quantising bf16 rows in the sender")
    ap.add_argument("--split", type=int, default=-1, metavar="P",
                    help="also measure the split dispatch with P private rows per "
                         "(destination, source) pair, alone and overlapped with a "
                         "shared-expert stand-in on a second stream")
    ap.add_argument("--graph", action="store_true",
                    help="capture K steps as one HIP graph and replay it (removes "
                         "launch overhead; matters for launch-bound small workloads)")
    ap.add_argument("--staged", action="store_true",
                    help="also time the materialised network write + unpack against the "
                         "fused receiver")
    ap.add_argument("--presum", action="store_true",
                    help="also measure the combine with partial sums on the expert side")
    ap.add_argument("--kv", action="store_true",
                    help="also measure the KV-block push (merged, per-block, staged)")
    ap.add_argument("--probe", default="", metavar="WORKLOADS",
                    help="only run the kernel-level probe (the sender back to back, after a "
                         "cache flush, and after a flush plus a read of the token rows, for "
                         "each listed workload; the copy probe at 0.5-3 GiB) and print it")
    ap.add_argument("--sender-probe", action="store_true",
                    help="measure what limits the quantising sender on the prefill workload "
                         "(public calls only) and print one JSON line")
    ap.add_argument("--pattern-probe", action="store_true",
                    help="measure the access shapes behind the kernels' designs (fills, "
                         "copies, the combine's 8:1 mix, memory-side cache reuse) with the "
                         "library's access-pattern probe and print one JSON line")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle CPU work for the baseline (0 = skip; the parity "
                         "check then runs the oracle once)")
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
    if args.probe:
        probe = measure_probe(ep, torch, np, W, [n for n in args.probe.split(",") if n],
                              Flusher(torch))
        print(json.dumps({"probe": probe}), flush=True)
        return 0
    if args.pattern_probe:
        print(json.dumps({"pattern_probe": measure_pattern_probe(ep, torch, np, W,
                                                                 Flusher(torch))}), flush=True)
        return 0
    if args.sender_probe:
        print(json.dumps({"sender_probe": measure_sender_probe(ep, torch, np, W, Flusher(torch))}),
              flush=True)
        return 0
    sh, wl, d, b, alpha = setup(ep, torch, np, W, args.config)
    quant = sh.payload == W.PAYLOAD_FP8_B128 and not args.prequantized
    x_bf16 = torch.from_numpy(wl.x_bf16.view(np.int16)).cuda() if quant else None
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    row_d = sum(ep.row_bytes(d, q) for q in range(ep.num_planes(d)))
    flush = Flusher(torch)

    def pack():
        if quant:
            ep.dispatch_pack_quant(d, x_bf16, b.plan_ws, b.send, sp)
        else:
            ep.dispatch_pack(d, b.x, b.plan_ws, b.send, sp)

    # expert outputs once (outside timing)
    b.status.zero_()
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

    def step(ev=None):
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Back to back: K steps queued between two events (events on every
    # `sample_every`-th step split dispatch from combine: an event record
    # between two kernels costs a few microseconds of GPU time).
    sampled = list(range(0, args.steps, args.sample_every))
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(events.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    b2b_us = t_start.elapsed_time(t_end) * 1e3 / args.steps
    steps_us = [ev[0].elapsed_time(ev[-1]) * 1e3 for ev in events.values()]
    dispatch_call_us = statistics.mean(ev[0].elapsed_time(ev[1]) for ev in events.values()) * 1e3

    # The timed region: K steps, each after a cache flush (outside its
    # events), as a model layer finds the caches after other kernels ran.
    t0 = time.perf_counter()
    flushed = time_flushed(torch, stream, step, args.steps, flush)
    wall_ms = (time.perf_counter() - t0) * 1e3
    us_per_step = statistics.mean(flushed)
    ms_per_step = us_per_step / 1e3
    status_after = int(b.status.item())

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
    # Per-stage times from the four separate calls, after the timed region;
    # the receiver kernel is the same launch in both forms of the step.
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
    ab = algorithmic_bytes(sh, row_d, quant)
    eff = ab["step"] / (ms_per_step * 1e-3) / 1e9

    # the dominant kernel against the roofline; beside its back-to-back
    # launches, the same kernel inside a step (the four-call stage loop: the
    # receiver right after the sender that wrote its rows)
    roof = dominant_roofline(ep, torch, d, b, sh, quant, x_bf16, ab, args.config, stream)
    dom = max(ab["stages"], key=lambda k: ab["stages"][k])
    in_step_ms = statistics.mean(per[dom])
    roof["in_step_us"] = round(in_step_ms * 1e3, 2)
    roof["in_step_frac"] = round(ab["stages"][dom] / (in_step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    roof["in_step_from"] = ("the same call inside the four-call steps of the stage loop, "
                            "between two HIP events")

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
    csrc = flush.a
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        ep.probe_copy(cdst, csrc, nbytes, sp)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        ep.probe_copy(cdst, csrc, nbytes, sp)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cdst

    split = None
    if args.split >= 0:
        split = measure_split(ep, torch, d, b, sh, args.split, args.steps, args.warmup)

    presum = None
    if args.presum:
        presum = measure_presum(ep, torch, np, d, b, sh, wl, alpha, args.steps, args.warmup)

    staged = None
    if args.staged:
        staged = measure_staged(ep, torch, d, sh, wl, max(args.steps // 5, 10), 3)

    kv = None
    if args.kv:
        kv = measure_kv(ep, torch, np, W)

    # The oracle: timed as the CPU baseline, and its result is what the
    # benchmarked buffers are compared with (the last step's plan tables,
    # send and grouped rows, and every combined token).
    import oracle
    cpu = None
    if args.cpu_budget > 0:
        base = cpu_baseline(sh, wl, args.cpu_budget, quant)
        oracle_out = base["out"]
        host = cpu_host()
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
            "threads": 1,
            "host_nproc": host["nproc"],
            "host_cpus_allowed": host["cpus_allowed"],
            "host_cpu_model": host["model"],
        }
        del base
    elif sh.n_ranks * sh.tokens * sh.hidden <= 1 << 25:
        oracle_out = oracle.run(wl, cap=ep.capacity(d))["out"]
    else:
        oracle_out = None     # sampled tokens and closed forms (bench_parity)
    # the plan, send rows and grouped rows of the last four-call pass (equal
    # by construction to the timed steps'), the combine of the last one
    parity = bench_parity(ep, torch, np, d, b, sh, wl, quant, oracle_out=oracle_out)
    parity["status_after_timed_steps"] = status_after

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
            "workload": describe(sh, W, quant),
            "parallelism": "ep (virtual ranks on one GPU)",
            "global_batch": sh.n_ranks * sh.tokens,
        },
        "timing": ("each of the K timed steps follows a 1 GiB fill and a 1 GiB read that "
                   "evict the L2s and the MALL, and is timed alone between two HIP events; "
                   "value and ms_per_step use the mean of the K steps"),
        "us_per_dispatch_combine": round(us_per_step, 2),
        "us_p10_p50_p90": pcts(np, flushed),
        "back_to_back_us_per_step": round(b2b_us, 2),
        "back_to_back_frac_of_hbm_peak": round(ab["step"] / b2b_us / 1e3 / HBM_PEAK_GBPS, 4),
        "us_per_virtual_rank": round(us_per_step / sh.n_ranks, 3),
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
        "stages_from": "the four separate calls, back to back, after the timed steps",
        "instrumented_step_us_p10_p50_p90": pcts(np, steps_us),
        "wall_ms": round(wall_ms, 3),
        "roofline": roof,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "parity": parity,
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

    # the other workloads, each under its own protocol, after freeing this one
    names = [n for n in args.configs.split(",") if n and n != args.config]
    if names:
        del b, x_bf16, alpha
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        res["configs"] = {}
        for n in names:
            res["configs"][n] = run_config(ep, torch, np, W, n, flush)
            gc.collect()
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Turn rocprofv3 outputs of bench.py runs into the summaries under profiles/.

Two summaries per workload:

  trace    rocprofv3 --kernel-trace --stats of one bench.py run ->
           profiles/<workload>_kernel_trace.md (calls and durations per kernel)
  traffic  two rocprofv3 --pmc runs of the same bench.py command, FETCH_SIZE
           in one and WRITE_SIZE in the other (one counter per run) ->
           profiles/<workload>_hbm_traffic.md and profiles/traffic_<workload>.json

Traffic calibration: bench.py's copy-ceiling leg launches the library's copy
probe on 1 GiB (1 GiB read, 1 GiB written per launch); each counter's reading
for that launch gives the factor that turns the counter into bytes. The JSON
records, per stage, the source hash of the kernels it was measured on;
bench.py only reports the traffic while the built kernels still hash the same.

A fourth tabulates `bench.py --pattern-probe` (fills, copies, the combine's
mix and memory-side cache reuse with the library's access-pattern probe).

A third summary tabulates counter runs of `bench.py --probe` (the senders
back to back, after a cache flush and after a flush plus a read of the token
rows; the copy probe at 0.5-3 GiB).

Usage (after the rocprofv3 runs, whose commands the summaries quote):
  python3 bench_profiles.py trace WORKLOAD STATS_CSV "BENCH_ARGS"
  python3 bench_profiles.py traffic WORKLOAD FETCH_CSV WRITE_CSV STATS_CSV "BENCH_ARGS"
  python3 bench_profiles.py probe TITLE WORKLOADS TIMING_JSON COUNTER_CSV...
  python3 bench_profiles.py pattern TIMING_JSON   (bench.py --pattern-probe)
"""
from __future__ import annotations

import collections
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")

# Kernels of each stage (the first one present is the stage's kernel; the
# plan stage sums its kernels).
STAGE_KERNELS = {
    "plan": [["plan_count_kernel", "plan_finalize_kernel"], ["plan_fused_kernel"]],
    "plan_local": [["plan_count_local_kernel"]],
    "pack": [["pack_gather_kernel<false, false>"], ["pack_fast1_kernel<14>"],
             ["pack_fast2_kernel<7, 1>"], ["pack_kernel"]],
    "pack_exchange": [["pack_gather_kernel<true, false>"], ["pack_exchange_kernel<14, 0>"]],
    "pack_quant": [["pack_quant_tok_kernel<false>"], ["pack_quant_kernel"]],
    "pack_quant_exchange": [["pack_quant_tok_kernel<true>"], ["pack_quant_exchange_kernel"]],
    "recv": [["recv_rows_kernel<false>"]],
    "combine": [["combine_kernel<7, 2, 2>"], ["combine_kernel<2, 7, 2>"]],
}
COPY_KERNEL = "probe_copy_kernel"


def short(name: str) -> str:
    n = name.replace("void ", "").replace("ep::(anonymous namespace)::", "")
    m = re.match(r"([\w:]+(<[^()]*>)?)", n)
    return m.group(1) if m else n[:60]


def command(args: str, extra: str) -> str:
    return ("cd /tmp && export TMPDIR=/tmp && rocprofv3 " + extra +
            " --output-format csv -d <out> -o run -- python3 /root/repo/bench.py " + args).strip()


def read_stats(path: str):
    rows = list(csv.DictReader(open(path)))
    return rows, {short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}


LIBRARY_PREFIXES = ("plan_", "pack_", "recv_", "combine_", "expert_", "presum", "kv_", "staged_",
                    "window_", "probe_")
B2B_RUN = 20


def back_to_back_runs(timeline):
    """Maximal runs of consecutive dispatches (in start order) of one library
    kernel on one grid, at least B2B_RUN long: [((name, grid), [durations])]."""
    runs, cur = [], None
    for _, key, t in sorted(timeline, key=lambda x: x[0]):
        if cur is not None and cur[0] == key:
            cur[1].append(t)
            continue
        if cur is not None and len(cur[1]) >= B2B_RUN and cur[0][0].startswith(LIBRARY_PREFIXES):
            runs.append(cur)
        cur = (key, [t])
    if cur is not None and len(cur[1]) >= B2B_RUN and cur[0][0].startswith(LIBRARY_PREFIXES):
        runs.append(cur)
    return runs


def trace(workload: str, stats_csv: str, args: str, out_dir: str = None) -> str:
    """Kernel statistics of one run; with the per-dispatch trace beside the
    statistics file, also grouped by kernel and grid size, which tells the
    workloads of one run apart (each launches its kernels on its own grid)."""
    rows, _ = read_stats(stats_csv)
    out = [f"# Kernel trace: {workload}", "",
           "Command (MI355X, one GPU), then this summary:", "", "```",
           command(args, "--kernel-trace --stats"),
           f"python3 bench_profiles.py trace {workload} <stats csv> \"{args}\"", "```", "",
           "rocprofv3 kernel statistics over every dispatch of the run: warm-up, back-to-back",
           "and flushed steps, the per-stage loop of four separate calls, 20 launches of the",
           "dominant kernel (of the headline and of each flushed workload in configs), the",
           "stand-in expert, the copy probe and the torch kernels that evict the caches",
           "between flushed steps.", "",
           "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    per_dispatch = os.path.join(os.path.dirname(stats_csv),
                                os.path.basename(stats_csv).replace("kernel_stats", "kernel_trace"))
    if os.path.exists(per_dispatch):
        groups = collections.OrderedDict()
        timeline = []   # (start, key, duration) of every dispatch, library or not
        for r in csv.DictReader(open(per_dispatch)):
            name = short(r["Kernel_Name"])
            key = (name, int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            timeline.append((int(r["Start_Timestamp"]), key, t))
            if not name.startswith(LIBRARY_PREFIXES):
                continue
            groups.setdefault(key, []).append(t)
        out += ["", "The library's kernels by launch grid (threads), in order of first launch:", "",
                "| kernel | grid threads | calls | avg us | min us | max us |",
                "|---|---|---|---|---|---|"]
        for (name, grid), ts in groups.items():
            out.append(f"| {name} | {grid} | {len(ts)} | {sum(ts) / len(ts):.2f} | "
                       f"{min(ts):.2f} | {max(ts):.2f} |")
        runs = back_to_back_runs(timeline)
        if runs:
            out += ["", f"Runs of at least {B2B_RUN} consecutive launches of one library kernel "
                    "on one grid, with no other dispatch between them (bench.py's roofline "
                    "loops: 20 launches of a workload's dominant kernel between two events), "
                    "in order:", "",
                    "| kernel | grid threads | launches | avg us | min us | max us |",
                    "|---|---|---|---|---|---|"]
            for (name, grid), ts in runs:
                out.append(f"| {name} | {grid} | {len(ts)} | {sum(ts) / len(ts):.2f} | "
                           f"{min(ts):.2f} | {max(ts):.2f} |")
    path = os.path.join(out_dir or PROFILES, f"{workload}_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return path


def counter_means(path: str) -> dict:
    """Mean counter value per dispatch, per kernel."""
    agg = collections.defaultdict(list)
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        i = int(r["Dispatch_Id"])
        per[i] += float(r["Counter_Value"])
        names[i] = short(r["Kernel_Name"])
    for i, v in per.items():
        agg[names[i]].append(v)
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic(workload: str, fetch_csv: str, write_csv: str, stats_csv: str, args: str,
            out_dir: str = None):
    import bench
    import ep_workloads as W

    fetch = counter_means(fetch_csv)
    write = counter_means(write_csv)
    _, avg = read_stats(stats_csv)
    copy_kib = (1 << 30) / 1024
    ff = copy_kib / fetch[COPY_KERNEL]
    wf = copy_kib / write[COPY_KERNEL]
    sh = W.CONFIGS[workload]
    quant = sh.payload == W.PAYLOAD_FP8_B128 and "--prequantized" not in args
    row_d = 2 * sh.hidden if sh.payload == W.PAYLOAD_BF16 else sh.hidden + 4 * (sh.hidden // 128)
    ab = bench.algorithmic_bytes(sh, row_d, quant)["stages"]
    alg = dict(ab)
    alg["plan_local"] = ab["plan"]
    alg["pack_exchange"] = ab["pack"]
    alg["pack_quant"] = ab["pack"]
    alg["pack_quant_exchange"] = ab["pack"]
    rec = {"workload": workload, "bench_args": args, "fetch_factor": round(ff, 4),
           "write_factor": round(wf, 4),
           "calibration": "probe_copy_kernel, 1 GiB read + 1 GiB written per launch",
           "stages": {}}
    md = [f"# HBM traffic per launch: {workload} workload", "",
          "Commands (MI355X, one GPU), one counter per run, then this summary:", "", "```",
          command(args, "--pmc FETCH_SIZE"), command(args, "--pmc WRITE_SIZE"),
          command(args, "--kernel-trace --stats"),
          f"python3 bench_profiles.py traffic {workload} <fetch csv> <write csv> <stats csv> "
          f"\"{args}\"", "```", "",
          "Calibration against the copy probe of the same run (1 GiB read, 1 GiB written per "
          f"launch): FETCH_SIZE reads {1 / ff:.3f}x the true bytes (factor {ff:.4f}), WRITE_SIZE "
          f"{1 / wf:.3f}x (factor {wf:.4f}). Counter values are means over every launch of the "
          "kernel in the run (warm and flushed alike); durations are the kernel trace's means.", "",
          "| stage | kernel | FETCH KiB (raw) | WRITE KiB (raw) | calibrated traffic bytes | "
          "algorithmic bytes | traffic / algorithmic | avg us (trace) | algorithmic GB/s |",
          "|---|---|---|---|---|---|---|---|---|"]
    for stage, options in STAGE_KERNELS.items():
        ks = next((o for o in options if all(k in fetch and k in write for k in o)), None)
        if ks is None:
            continue
        if stage in ("pack", "pack_exchange") and quant:
            continue
        fk = sum(fetch[k] for k in ks)
        wk = sum(write[k] for k in ks)
        t = int(fk * 1024 * ff + wk * 1024 * wf)
        us = sum(avg.get(k, float("nan")) for k in ks)
        a = alg[stage]
        rec["stages"][stage] = {
            "kernels": ks, "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
            "traffic_bytes": t, "algorithmic_bytes": a,
            "traffic_over_algorithmic": round(t / a, 4), "avg_us": round(us, 2),
            "sources": bench.STAGE_SOURCES[stage],
            "source_sha256_16": bench.kernel_source_hash(bench.STAGE_SOURCES[stage])}
        md.append(f"| {stage} | {' + '.join(ks)} | {fk:.1f} | {wk:.1f} | {t} | {a} | "
                  f"{t / a:.4f} | {us:.2f} | {a / us / 1e3:.1f} |")
    md += ["",
           "The plan stages' algorithmic bytes count only the routing ids; their traffic "
           "includes the plan tables they write (and, for plan_local, the token rows it "
           "touches for the sender).",
           "traffic_" + workload + ".json holds these figures with a source hash per stage; "
           "bench.py reports a stage's traffic only while its kernels hash the same."]
    p_md = os.path.join(out_dir or PROFILES, f"{workload}_hbm_traffic.md")
    p_js = os.path.join(out_dir or PROFILES, f"traffic_{workload}.json")
    with open(p_md, "w") as fh:
        fh.write("\n".join(md) + "\n")
    with open(p_js, "w") as fh:
        json.dump(rec, fh, indent=1)
    return p_md, p_js


SENDER_KERNELS = ("pack_gather_kernel<false, false>", "pack_fast1_kernel<14>",
                  "pack_fast2_kernel<7, 1>", "pack_kernel", "pack_quant_tok_kernel<false>",
                  "pack_quant_kernel")


def probe(title: str, workloads: str, timing_json: str, counter_csvs: list) -> str:
    """Counter summary of `bench.py --probe WORKLOADS` runs: per workload the
    sender launches in the probe's order (3 untimed steps, 5 back to back, 5
    after a cache flush, 5 after a flush and a read of the token rows), then
    the copy probe (3 launches each of 0.5, 1, 2, 3 GiB); per phase the mean of
    each counter over the sender's launches, beside the event timings of an
    unprofiled run."""
    names = [n for n in workloads.split(",") if n]
    with open(timing_json) as fh:
        timing = json.loads(fh.read().strip().splitlines()[-1])["probe"]
    phases = [("back to back", 3, 8), ("after flush", 8, 13), ("after flush + token read", 13, 18)]
    table = collections.defaultdict(dict)   # (row label) -> counter -> value
    counters = []
    for path in counter_csvs:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        kname = {}
        for r in csv.DictReader(open(path)):
            i = int(r["Dispatch_Id"])
            per[i][r["Counter_Name"]] += float(r["Counter_Value"])
            kname[i] = short(r["Kernel_Name"])
        ids = sorted(per)
        senders = [i for i in ids if kname[i] in SENDER_KERNELS]
        copies = [i for i in ids if kname[i] == COPY_KERNEL]
        cn = sorted({c for i in ids for c in per[i]})
        counters += [c for c in cn if c not in counters]
        for w, name in enumerate(names):
            mine = senders[18 * w:18 * (w + 1)]
            for label, a, b in phases:
                for c in cn:
                    v = [per[i][c] for i in mine[a:b]]
                    table[(name, label)][c] = sum(v) / len(v)
        for j, gib in enumerate(("0.5GiB", "1GiB", "2GiB", "3GiB")):
            for c in cn:
                v = [per[i][c] for i in copies[3 * j:3 * j + 3]]
                table[("copy " + gib, "")][c] = sum(v) / len(v)
    head = ["# " + title, "", "Commands (MI355X, one GPU): the event timings come from the first "
            "run; each counter set from its own rocprofv3 run of the same probe; then this "
            "summary.", "", "```", f"python3 /root/repo/bench.py --probe {workloads}"]
    for c in counter_csvs:
        sets = sorted({r["Counter_Name"] for r in csv.DictReader(open(c))})
        head.append(command(f"--probe {workloads}", "--pmc " + " ".join(sets)))
    head += [f"python3 bench_profiles.py probe \"{title}\" {workloads} <timing json> "
             "<counter csv> ...", "```", "",
             "Event timings (us, median of 5 steps of the four separate calls, each stage "
             "between two events):", "",
             "| workload | stage | algorithmic bytes | back to back | after flush | "
             "after flush + token read |", "|---|---|---|---|---|---|"]
    for name in names:
        t = timing[name]
        for st, key in (("plan", "plan"), ("sender", "pack"), ("recv", "recv"),
                        ("combine", "combine")):
            label = t["sender"] if st == "sender" else st
            head.append(f"| {name} | {label} | {t['algorithmic_bytes'][key]} | "
                        f"{t['back_to_back_us'][st]} | {t['after_flush_us'][st]} | "
                        f"{t['after_flush_and_token_read_us'][st]} |")
    head += ["", "Copy probe (each launch alone; read + write bytes):", "",
             "| size | us (3 launches) | TB/s |", "|---|---|---|"]
    for gib, c in timing["copy_probe"].items():
        head.append(f"| {gib} | {c['us']} | {c['TBps']} |")
    head += ["", "Counters, mean per launch (the `_sum` counters summed over instances):", "",
             "| launches | " + " | ".join(counters) + " |",
             "|---|" + "---|" * len(counters)]
    for (w, label), vals in table.items():
        row = f"{w} {label}".strip()
        head.append(f"| {row} | " + " | ".join(f"{vals.get(c, float('nan')):.4g}"
                                                for c in counters) + " |")
    path = os.path.join(PROFILES, title.lower().replace(" ", "_").replace(",", "") + ".md")
    with open(path, "w") as fh:
        fh.write("\n".join(head) + "\n")
    return path


def pattern(timing_json: str, out_dir: str = None) -> str:
    """Tables of one `bench.py --pattern-probe` run -> profiles/access_pattern_probe.md."""
    with open(timing_json) as fh:
        t = json.loads(fh.read().strip().splitlines()[-1])["pattern_probe"]

    def cell(f):
        return f"{f['us']} ({f['TBps']})"

    out = ["# Access-pattern probe", "",
           "The access shapes the sender, receiver and combine were chosen on, measured with",
           "the library's `ep_probe_pattern` (each wave moves one piece of the output, 16",
           "bytes per lane at a time, non-temporal stores). Each figure is the median of 5",
           "launches, each alone between two HIP events, back to back unless stated: µs",
           "(TB/s of the bytes given).", "",
           "Commands (MI355X, one GPU):", "", "```",
           "python3 /root/repo/bench.py --pattern-probe > <timing json>",
           "python3 bench_profiles.py pattern <timing json>", "```", "",
           "## Fills of 1 GiB (bytes written)", "", "| shape | µs (TB/s) |", "|---|---|"]
    for k, f in t["fill_1GiB"].items():
        out.append(f"| {k.replace('_', ' ')} | {cell(f)} |")
    if "copy_1GiB" in t:
        out += ["", "## Copies of 1 GiB (bytes read + written)", "", "| copy | µs (TB/s) |",
                "|---|---|"]
        labels = {"1KB_per_wave_nt_loads": "access-pattern probe, 1 KB per wave, nt loads",
                  "ep_probe_copy_7KB_per_wave": "`ep_probe_copy` (7 KB per wave)",
                  "torch_copy_": "torch `copy_`"}
        for k, f in t["copy_1GiB"].items():
            out.append(f"| {labels.get(k, k)} | {cell(f)} |")
    c = t["copy_decode_size"]
    b = c["bytes"]
    out += ["", "## Copies of the decode size: 32768 rows of 14 KB written", "",
            f"Bytes: {b['linear_and_permuted']} (read + write) for the linear and permuted "
            f"copies; {b['sender_like']} (token rows once + writes) for the sender-like ones, "
            "which read each of 4096 token rows 8 times in the decode routing's send order.",
            "", "| per wave | linear (nt loads) | rows permuted (nt) | sender-like: cached, XCD "
            "order | cached | nt, XCD order |", "|---|---|---|---|---|---|"]
    for k, f in c["figures"].items():
        out.append(f"| {k.split('_')[0]} | {cell(f['linear'])} | {cell(f['rows_permuted'])} | "
                   f"{cell(f['sender_like_cached_xcd'])} | {cell(f['sender_like_cached'])} | "
                   f"{cell(f['sender_like_nt_xcd'])} |")
    if "receiver_orders_decode_size" in t:
        ro = t["receiver_orders_decode_size"]
        out += ["", "## The receiver's row pairs at the decode size", "",
                f"The decode routing's 32768 (send row, grouped row) pairs, {ro['bytes']} bytes "
                "(read + write), 1 KB per wave, non-temporal loads. Receive order writes the "
                "grouped rows in order and reads the send rows the table names (the library's "
                "receiver); send order reads the send rows in order and scatters each to its "
                "grouped row.", "", "| order | µs (TB/s) |", "|---|---|",
                f"| receive order | {cell(ro['receive_order'])} |",
                f"| send order | {cell(ro['send_order'])} |"]
    if "workgroup_size_decode_size" in t:
        wg = t["workgroup_size_decode_size"]
        labels = {"linear_copy": "linear copy", "rows_permuted": "rows permuted",
                  "receiver_pairs_receive_order": "the receiver's pairs, receive order",
                  "combine_mix_8_in_flight": "the combine's 8:1 mix, 8 rows in flight",
                  "fill": "fill", "read": "read"}
        out += ["", "## Workgroups of four waves against one at the decode size", "",
                "The same shapes, 1 KB per wave, non-temporal loads; copies move 939524096 "
                "bytes (read + write), the mix 528482304, fill and read 469762048.", "",
                "| shape | four waves | one wave |", "|---|---|---|"]
        for k in wg["four_waves"]:
            out.append(f"| {labels.get(k, k)} | {cell(wg['four_waves'][k])} | "
                       f"{cell(wg['one_wave'][k])} |")
    m = t["combine_mix_decode_size"]
    out += ["", "## The combine's 8:1 mix at the decode size", "",
            f"4096 rows of 14 KB, each the xor of 8 rows from 8 linear regions: {m['bytes']} "
            "bytes (470 MB read, 59 MB written); the read-only lines read the 470 MB alone.",
            "", "| shape | µs (TB/s) |", "|---|---|"]
    for k, f in m["figures"].items():
        out.append(f"| {k.replace('_', ' ')} | {cell(f)} |")
    out += ["", "## Reuse from the memory-side cache", "",
            "A buffer read with 1 KB per wave right after a fill of the same bytes, right "
            "after a read of them, and after a flush (1 GiB fill + 1 GiB read).", "",
            "| size | loads | after fill | after read | after flush |", "|---|---|---|---|---|"]
    for size, e in t["mall_reuse"].items():
        for loads in ("nt", "cached"):
            out.append(f"| {size} | {loads} | {cell(e[loads + '_after_fill'])} | "
                       f"{cell(e[loads + '_after_read'])} | {cell(e[loads + '_after_flush'])} |")
    if "sender_orders_by_source_size" in t:
        out += ["", "## The sender's orders by bytes per source", "",
                "8 sources of T token rows of 14 KB, top-8 of 256 experts, uniform routing; "
                "bytes: the token rows once plus the 8 T send rows of each source. Send order: "
                "the gather (cached loads, XCD renumbering, 1 KB per wave). Token order: a "
                "scatter (each token row read once with non-temporal loads and written to its "
                "8 send rows).", "",
                "| per source | T | send order, 1 KB | token order, 1 KB | token order, 14 KB |",
                "|---|---|---|---|---|"]
        for k, e in t["sender_orders_by_source_size"].items():
            out.append(f"| {k.split('_')[0]} | {e['tokens']} | {cell(e['send_order_1KB'])} | "
                       f"{cell(e['token_order_1KB'])} | {cell(e['token_order_14KB'])} |")
    path = os.path.join(out_dir or PROFILES, "access_pattern_probe.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return path


def main(argv) -> int:
    if len(argv) >= 4 and argv[0] == "trace":
        print(trace(argv[1], argv[2], argv[3]))
        return 0
    if len(argv) >= 6 and argv[0] == "traffic":
        print(*traffic(argv[1], argv[2], argv[3], argv[4], argv[5]))
        return 0
    if len(argv) >= 5 and argv[0] == "probe":
        print(probe(argv[1], argv[2], argv[3], argv[4:]))
        return 0
    if len(argv) >= 2 and argv[0] == "pattern":
        print(pattern(argv[1]))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

"""bench_profiles.py, the tool that turns rocprofv3 output into the summaries
under profiles/, on small synthetic CSVs (no GPU): the traffic calibration
against the copy probe, the per-grid grouping of the kernel trace, and the
access-pattern tables."""
import csv
import json
import os

import bench
import bench_profiles as bp
import ep_workloads as W

GiB_KiB = (1 << 30) // 1024


def write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def counters(path, counter, per_dispatch):
    """per_dispatch: [(dispatch id, kernel name, [values of the counter's instances])]."""
    rows = [(i, name, counter, v) for i, name, vals in per_dispatch for v in vals]
    write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def stats(path, kernels):
    write_csv(path, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [(n, c, a, a, a, p) for n, c, a, p in kernels])


def test_traffic_is_calibrated_by_the_copy_probe(tmp_path):
    copy = "void ep::(anonymous namespace)::probe_copy_kernel(uint4 const*, uint4*, long)"
    recv = "void ep::(anonymous namespace)::recv_rows_kernel<false>(ep::RecvArgs)"
    comb = "void ep::(anonymous namespace)::combine_kernel<7, 2, 2>(unsigned short const*)"
    # FETCH_SIZE reads half the bytes (two instances per dispatch), WRITE_SIZE all of them.
    counters(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, copy, [GiB_KiB / 4, GiB_KiB / 4]),
        (2, recv, [100000.0, 130000.0]), (3, recv, [120000.0, 110000.0]),
        (4, comb, [200000.0, 0.0])])
    counters(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, copy, [GiB_KiB / 2, GiB_KiB / 2]),
        (2, recv, [450000.0]), (3, recv, [470000.0]), (4, comb, [57000.0])])
    stats(tmp_path / "s.csv", [(recv, 2, 149000.0, 60.0), (comb, 1, 89000.0, 30.0),
                               (copy, 1, 340000.0, 10.0)])
    md, js = bp.traffic("decode", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                        str(tmp_path / "s.csv"), "--config decode", out_dir=str(tmp_path))
    rec = json.load(open(js))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    r = rec["stages"]["recv"]
    assert r["fetch_kib_raw"] == 230000.0 and r["write_kib_raw"] == 460000.0
    assert r["traffic_bytes"] == 230000 * 1024 * 2 + 460000 * 1024
    sh = W.CONFIGS["decode"]
    alg = bench.algorithmic_bytes(sh, 2 * sh.hidden, False)["stages"]
    assert r["algorithmic_bytes"] == alg["recv"] == 2 * 32768 * 14336
    assert r["avg_us"] == 149.0
    assert r["source_sha256_16"] == bench.kernel_source_hash(bench.STAGE_SOURCES["recv"])
    assert rec["stages"]["combine"]["traffic_bytes"] == 200000 * 1024 * 2 + 57000 * 1024
    assert "plan" not in rec["stages"]       # no plan kernels in these CSVs
    assert os.path.basename(md) == "decode_hbm_traffic.md"
    assert "| recv | recv_rows_kernel<false> | 230000.0 | 460000.0 |" in open(md).read()


def test_trace_groups_library_kernels_by_grid(tmp_path):
    recv = "void ep::(anonymous namespace)::recv_rows_kernel<false>(ep::RecvArgs)"
    torch_k = "void at::native::vectorized_elementwise_kernel<4>(int)"
    stats(tmp_path / "run_kernel_stats.csv", [(recv, 3, 100000.0, 90.0),
                                              (torch_k, 1, 5000.0, 10.0)])
    rows = [(recv, 4096, 0, 10000), (recv, 4096, 20000, 32000), (recv, 8192, 40000, 140000),
            (torch_k, 256, 150000, 155000)]
    write_csv(tmp_path / "run_kernel_trace.csv",
              ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
               "End_Timestamp"], [(n, g, 1, 1, a, b) for n, g, a, b in rows])
    path = bp.trace("toy", str(tmp_path / "run_kernel_stats.csv"), "--config toy",
                    out_dir=str(tmp_path))
    text = open(path).read()
    assert "| recv_rows_kernel<false> | 4096 | 2 | 11.00 | 10.00 | 12.00 |" in text
    assert "| recv_rows_kernel<false> | 8192 | 1 | 100.00 | 100.00 | 100.00 |" in text
    assert "vectorized_elementwise_kernel<4> | 256" not in text   # torch kernels: stats only


def test_pattern_tables_render_every_section(tmp_path):
    f = {"us": 10.0, "TBps": 1.0}
    copies = {k: f for k in ("linear", "rows_permuted", "sender_like_cached_xcd",
                             "sender_like_cached", "sender_like_nt_xcd")}
    reuse = {f"{l}_after_{w}": f for l in ("nt", "cached") for w in ("fill", "read", "flush")}
    t = {"fill_1GiB": {"1KB_per_wave": f},
         "copy_1GiB": {"1KB_per_wave_nt_loads": f, "ep_probe_copy_7KB_per_wave": f,
                       "torch_copy_": f},
         "copy_decode_size": {"bytes": {"linear_and_permuted": 1, "sender_like": 2},
                              "figures": {"1KB_per_wave": copies}},
         "receiver_orders_decode_size": {"bytes": 3, "receive_order": f, "send_order": f},
         "workgroup_size_decode_size": {"four_waves": {"linear_copy": f, "fill": f},
                                        "one_wave": {"linear_copy": f, "fill": f}},
         "combine_mix_decode_size": {"bytes": 4, "figures": {"read_only_1KB_nt": f}},
         "mall_reuse": {"32MB": reuse},
         "sender_orders_by_source_size": {"1.8MB_per_source": {
             "tokens": 128, "send_order_1KB": f, "token_order_1KB": f, "token_order_14KB": f}}}
    (tmp_path / "p.json").write_text("some log line\n" + json.dumps({"pattern_probe": t}) + "\n")
    text = open(bp.pattern(str(tmp_path / "p.json"), out_dir=str(tmp_path))).read()
    for head in ("## Fills of 1 GiB", "## Copies of 1 GiB", "## Copies of the decode size",
                 "## The receiver's row pairs", "## Workgroups of four waves against one",
                 "## The combine's 8:1 mix",
                 "## Reuse from the memory-side cache", "## The sender's orders"):
        assert head in text
    assert "| 1KB | 10.0 (1.0) |" in text
    assert "| linear copy | 10.0 (1.0) | 10.0 (1.0) |" in text
    assert "| 32MB | cached | 10.0 (1.0) | 10.0 (1.0) | 10.0 (1.0) |" in text
    assert "| 1.8MB | 128 | 10.0 (1.0) |" in text


def test_trace_lists_back_to_back_runs(tmp_path):
    """The roofline loop's launches (20 or more of one kernel and grid with no
    other dispatch between them) are tabulated apart from the in-step ones."""
    recv = "void ep::(anonymous namespace)::recv_rows_kernel<false>(ep::RecvArgs)"
    pack = "void ep::(anonymous namespace)::pack_gather_kernel<true, false>(ep::GatherArgs)"
    stats(tmp_path / "run_kernel_stats.csv", [(recv, 23, 100000.0, 90.0), (pack, 3, 5000.0, 10.0)])
    rows, t = [], 0
    for k in range(2):                      # two steps: pack then recv (150 us)
        rows += [(pack, 4096, t, t + 70000), (recv, 4096, t + 80000, t + 230000)]
        t += 300000
    rows.append((pack, 4096, t, t + 70000))  # the loop's own plan and sender pass
    t += 80000
    for k in range(21):                     # the roofline loop: 21 launches of 140 us
        rows.append((recv, 4096, t, t + 140000))
        t += 150000
    rows.append((recv, 8192, t, t + 50000))  # another grid right after: not part of the run
    write_csv(tmp_path / "run_kernel_trace.csv",
              ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
               "End_Timestamp"], [(n, g, 1, 1, a, b) for n, g, a, b in rows[::-1]])
    text = open(bp.trace("toy", str(tmp_path / "run_kernel_stats.csv"), "--config toy",
                         out_dir=str(tmp_path))).read()
    assert "| recv_rows_kernel<false> | 4096 | 23 | 140.87 | 140.00 | 150.00 |" in text
    assert "| recv_rows_kernel<false> | 4096 | 21 | 140.00 | 140.00 | 140.00 |" in text
    assert text.count("| 21 | 140.00 |") == 1

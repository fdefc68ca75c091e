"""Plant plausible mistakes in a copy of the oracle and check a pin fails.

Each mutation edits the oracle's C source text in a temporary directory
(a dropped term, an off-by-one, a wrong index, a swapped operand), builds
it and runs the pins against it in a child process (a mutant may write
out of bounds; a crash counts as noticed). A mutation that no pin notices
would mean the pins cannot vouch for that part of the oracle.
"""
import ctypes
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, HERE)
import test_oracle_pins as pins  # noqa: E402

MUTATIONS = {
    "rank_dropped": ("send_pos[i] = send_off[(size_t)s * (E + 1) + e] + seen[e];",
                     "send_pos[i] = send_off[(size_t)s * (E + 1) + e];"),
    "send_scan_inclusive": ("so[e + 1] = so[e] + cnt[(size_t)s * E + e];",
                            "so[e + 1] = so[e] + cnt[(size_t)s * E + e] + (e == 0);"),
    "earlier_sources_inclusive": ("for (int s2 = 0; s2 < s; ++s2)\n                    before += cnt[(size_t)s2 * E + e];\n                int64_t rank",
                                  "for (int s2 = 0; s2 <= s; ++s2)\n                    before += cnt[(size_t)s2 * E + e];\n                int64_t rank"),
    "owner_interleaved": ("int d = e / L, j = e % L;", "int d = e % N, j = e / N;"),
    "recv_off_not_cumulative": ("ro[s + 1] = ro[s] + rows;", "ro[s + 1] = rows;"),
    "grp_off_wrong_column": ("col += cnt[(size_t)s * E + d * L + j];",
                             "col += cnt[(size_t)s * E + j];"),
    "capacity_off_by_one": ("grp_pos[i] = (g < cap) ? (int32_t)g : -1;",
                            "grp_pos[i] = (g <= cap) ? (int32_t)g : -1;"),
    "capacity_flag_inclusive": ("if ((int64_t)ro[N] > cap)", "if ((int64_t)ro[N] >= cap)"),
    "combine_weights_reversed": ("acc += (double)w[k] * (double)oracle_bf16_to_f32(rows[k][h]);",
                                 "acc += (double)w[R - 1 - k] * (double)oracle_bf16_to_f32(rows[k][h]);"),
    "combine_single_precision": ("double acc = 0.0;", "float acc = 0.0f;"),
    "bf16_quantum": ("double quantum = ldexp(1.0, e - 7);", "double quantum = ldexp(1.0, e - 8);"),
    "bf16_truncates": ("double r = nearbyint(n);", "double r = floor(n);"),
    "bf16_drops_sign": ("return sign | (uint16_t)((u >> 16) & 0x7FFF);",
                        "return (uint16_t)((u >> 16) & 0x7FFF);"),
    "e4m3_bias": ("v = ldexp(1.0 + (double)m / 8.0, ex - 7);",
                  "v = ldexp(1.0 + (double)m / 8.0, ex - 8);"),
    "e4m3_subnormal": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "pack_wrong_token": ("x + ((size_t)s * T + t) * row, (size_t)row);",
                         "x + ((size_t)s * T + (T - 1 - t)) * row, (size_t)row);"),
    "unpack_expert_offset_dropped": ("int64_t src = seg + in_seg + i;", "int64_t src = seg + i;"),
    "expert_scale_ignored": ("float v = oracle_bf16_to_f32(in[h]) * alpha[e];",
                             "float v = oracle_bf16_to_f32(in[h]) * alpha[0];"),
    "dequant_block": ("float v = oracle_e4m3_to_f32(codes[h]) * scales[h / 128];",
                      "float v = oracle_e4m3_to_f32(codes[h]) * scales[h / 256];"),
    "bound_min": ("int64_t m = R > L ? R : L;", "int64_t m = R < L ? R : L;"),
    "e4m3_ties_odd": ("(d == best_d && (c & 1) == 0 && (best & 1) != 0)",
                      "(d == best_d && (c & 1) != 0 && (best & 1) == 0)"),
    "e4m3_sign_dropped": ("    return sign | best;", "    return best;"),
    "quant_scale_max": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                        "float scale = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    "quant_zero_scale": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                         "float scale = amax > 0.0f ? amax / 448.0f : 0.5f;"),
    "presum_rank_ignored": ("for (int k2 = k; k2 < R; ++k2)\n                if (rows[k2] && rank[k2] == rank[k])",
                            "for (int k2 = k; k2 < R; ++k2)\n                if (rows[k2])"),
    "presum_leader_weight": ("acc = fmaf(w[k2], oracle_bf16_to_f32(rows[k2][h]), acc);",
                             "acc = fmaf(w[k], oracle_bf16_to_f32(rows[k2][h]), acc);"),
    "presum_leader_is_last": ("        int leader = 1;\n        for (int k2 = 0; k2 < k; ++k2)",
                              "        int leader = 1;\n        for (int k2 = k + 1; k2 < R; ++k2)"),
    "presum_groups_by_expert": ("rank[k] = e / L;", "rank[k] = e;"),
    "kv_src_only_contiguity": ("if (m > 0 && src_off[m - 1] + bytes[m - 1] == a &&\n            dst_off[m - 1] + bytes[m - 1] == b)",
                               "if (m > 0 && src_off[m - 1] + bytes[m - 1] == a)"),
    "kv_block_slot_dropped": ("return ((int64_t)blocks[i / bs] * bs + i % bs) * tok;",
                              "return ((int64_t)blocks[i / bs] * bs) * tok;"),
    "kv_copy_rank_stride": ("memcpy(dst + r * dst_rank_bytes + dst_off[j],",
                            "memcpy(dst + dst_off[j],"),
    "e4m3_inf_not_saturated": ("    if (isinf(a))\n        return sign | 0x7E;", ""),
    "quant_nan_in_amax": ("            if (a > amax)\n                amax = a;",
                          "            if (!(a <= amax))\n                amax = a;"),
    "quant_nan_not_nan_code": ("    if (isnan(v))\n        return 0x7F;\n    uint8_t sign",
                               "    if (isnan(v))\n        return 0x00;\n    uint8_t sign"),
    "quant_pack_source_offset_dropped": ("size_t row = (size_t)s * T * R + (size_t)p;",
                                         "size_t row = (size_t)p;"),
    "quant_pack_scale_row": ("memcpy(scales + row * (H / 128), qs,",
                             "memcpy(scales + (size_t)p * (H / 128), qs,"),
    "quant_pack_wrong_token": ("oracle_quantize_b128(H, x + ((size_t)s * T + t) * H, qc, qs);",
                               "oracle_quantize_b128(H, x + ((size_t)s * T + (T - 1 - t)) * H, qc, qs);"),
    "unpack_overflow_rows_left_stale": ("memset(grouped + ((size_t)d * cap + dst) * row, 0, (size_t)row);",
                                        ";"),
    "quant_block_size": ("float a = fabsf(oracle_bf16_to_f32(x[b * 128 + i]));",
                         "float a = fabsf(oracle_bf16_to_f32(x[b * 128 + (i & 63)]));"),
}


def _pin_checks():
    """The pins, as plain callables (parametrised ones with one case each)."""
    return [
        pins.test_f32_to_bf16_matches_torch,
        pins.test_f64_to_bf16_matches_brute_force,
        pins.test_e4m3_decode_matches_torch,
        pins.test_recv_bound_golden,
        pins.test_plan_hand_worked_example,
        pins.test_payload_hand_worked_example,
        lambda: pins.test_plan_matches_brute_force(3, 7, 9, 3, True, 1),
        lambda: pins.test_plan_matches_brute_force(2, 6, 8, 4, False, 4),
        lambda: pins.test_plan_matches_stable_argsort("tiny"),
        lambda: pins.test_plan_matches_stable_argsort("worst"),
        lambda: pins.test_plan_invariants("tiny_zipf"),
        pins.test_plan_bad_expert_and_capacity,
        lambda: pins.test_grouped_rows_are_source_rows("tiny_zipf"),
        lambda: pins.test_combine_identity_closed_form("tiny"),
        pins.test_combine_exact_brute_force_scale_expert,
        pins.test_expert_dequant_matches_torch,
        pins.test_combine_token_rounds_once,
        pins.test_f32_to_e4m3_matches_torch_including_ties,
        pins.test_quantize_b128_matches_generator_quantiser,
        pins.test_quantize_b128_roundtrip_error_bound,
        pins.test_f32_to_e4m3_saturates_infinities,
        pins.test_quantize_b128_non_finite_blocks,
        pins.test_dispatch_pack_quant_is_quantise_then_place,
        pins.test_staged_overflow_rows_are_source_rows_or_zeros,
        pins.test_presum_groups_by_rank_and_rounds_each_partial,
        pins.test_presum_adds_partials_in_slot_order,
        pins.test_presum_single_choice_is_the_rounded_product,
        pins.test_presum_one_rank_exact_sums_equal_the_plain_combine,
        pins.test_presum_partial_rows_sit_at_group_leaders,
        pins.test_kv_regions_hand_worked_example,
        lambda: pins.test_kv_regions_equal_block_sizes_count_block_runs(0),
        pins.test_kv_regions_identity_tables_are_one_region,
        lambda: pins.test_kv_copy_puts_each_token_where_the_tables_say(4, 16),
    ]


def _build_variant(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation {name} does not apply"
    mutated = src.replace(old, new, 1)
    d = tmp_path / name
    d.mkdir()
    c = d / "ep_oracle.c"
    c.write_text(mutated)
    (d / "ep_oracle.h").write_text(open(os.path.join(os.path.dirname(oracle._SRC), "ep_oracle.h")).read())
    so = d / "liboracle.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-w", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


def count_failures(lib_path=None):
    """Run every pin check (against `lib_path` if given); return #failed."""
    if lib_path is not None:
        L = ctypes.CDLL(lib_path)
        oracle._declare(L)
        oracle._lib = L
    failures = 0
    for chk in _pin_checks():
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


def test_clean_oracle_passes_every_check():
    assert count_failures() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    so = _build_variant(tmp_path, name, old, new)
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle_mutations as m; "
            "print('FAILED_PINS', m.count_failures(%r))" % (ROOT, HERE, so))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return                      # the mutant crashed a pin: noticed
    n = int(r.stdout.split("FAILED_PINS")[-1].split()[0])
    assert n > 0, f"no pin notices mutation {name}"

"""The benchmark's contract pieces that need no GPU."""
import os
import subprocess
import sys

import pytest

import ep_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_algorithmic_bytes_follow_the_step_formula():
    """Per-stage bytes sum to N T row_d + 3 N T R row_d + N T R row_c +
    N T row_c + 8 N T R: 1,996,750,848 B at decode shapes."""
    sh = W.CONFIGS["decode"]
    ab = bench.algorithmic_bytes(sh, 2 * sh.hidden, quant=False)
    N, T, R, H = sh.n_ranks, sh.tokens, sh.topk, sh.hidden
    row = 2 * H
    assert ab["step"] == N * T * row + 3 * N * T * R * row + N * T * R * row + N * T * row + 8 * N * T * R
    assert ab["step"] == 1_996_750_848
    assert ab["stages"]["recv"] == 2 * N * T * R * row


def test_quantising_sender_reads_bf16_rows():
    sh = W.CONFIGS["decode_fp8"]
    row_d = sh.hidden + 4 * (sh.hidden // 128)
    plain = bench.algorithmic_bytes(sh, row_d, quant=False)["stages"]["pack"]
    quant = bench.algorithmic_bytes(sh, row_d, quant=True)["stages"]["pack"]
    assert quant - plain == sh.n_ranks * sh.tokens * (2 * sh.hidden - row_d)


@pytest.mark.parametrize("stage", sorted(bench.STAGE_SOURCES))
def test_stage_sources_exist(stage):
    assert len(bench.kernel_source_hash(bench.STAGE_SOURCES[stage])) == 16

"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the
algorithmic byte and flop counts the roofline fractions divide by, and the
rule that a counter summary is used only when it was taken on the current
kernel sources."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_expert_bytes_of_the_decode_layer():
    # gate, up, down at hidden 4096 / inter 1536: codes 4 bits per weight plus
    # one f32 scale per 64 inputs
    w = 3 * 4096 * 1536
    assert bench.EXPERT_BYTES == w // 2 + w // 64 * 4 == 10_616_832
    assert bench.expert_bytes(64) == bench.EXPERT_BYTES
    assert bench.expert_bytes(32) == bench.EXPERT_BYTES + w // 64 * 4
    assert bench.expert_bytes(128) == bench.EXPERT_BYTES - w // 128 * 4


def test_decode_alg_counts_unique_valid_experts_and_valid_pairs():
    ids = torch.tensor([[0, 1, 1, 200, 5, 5, 5, 7], [-1, 3, 0, 2, 9, 9, 9, 9]])
    nbytes, flops, roof = bench.decode_alg(ids, 2)
    uniq = len({0, 1, 5, 7, 3, 2, 9})
    pairs = 16 - 2
    assert nbytes == uniq * bench.EXPERT_BYTES + 2 * 4096 * 4 * 2 + 2 * 8 * 8
    assert flops == 2.0 * pairs * 3 * 4096 * 1536
    assert roof == max(nbytes / bench.HBM_PEAK, flops / bench.F32_PEAK)


def test_prefill_alg_counts_gate_up_as_two_thirds():
    ids = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7], [0, 0, 1, 1, -3, 130, 2, 2]])
    nbytes, flops, gu, roof = bench.prefill_alg(ids, 2)
    assert flops == 2.0 * 14 * 3 * 4096 * 1536
    assert gu == flops * 2 / 3
    assert nbytes == 8 * bench.EXPERT_BYTES + 2 * 4096 * 2 + 2 * 4096 * 4 + 2 * 8 * 8
    assert roof == max(nbytes / bench.HBM_PEAK, flops / bench.BF16_PEAK)


def test_traffic_needs_the_current_sources(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// not the kernel the counters were taken on\n")
    assert bench.load_traffic([str(src)]) is None
    a = bench.source_hash([str(src)])
    src.write_text("// changed\n")
    assert bench.source_hash([str(src)]) != a


def test_expert_bytes_of_the_large_layer():
    # hidden 6144 / inter 2048: the pages' "19 megs" packed, "22 megs" with scales
    assert bench.layer_bytes_per_expert(6144, 2048) == 21_233_664
    assert bench.layer_bytes_per_expert(4096, 1536) == bench.EXPERT_BYTES


def test_decode_gateup_bytes_count_gate_and_up_once_per_expert():
    ids = torch.tensor([[0, 1, 1, 200], [1, -1, 0, 3]])
    gu = 1536 * 4096 // 2 + 1536 * 64 * 4
    assert bench.decode_gateup_bytes(ids, 2) == 3 * 2 * gu + 2 * 4096 * 4

"""CPU checks of the benchmark's accounting: the flop and byte counts it divides
by, and its refusal of more than one GPU."""
import subprocess
import sys
import os

import numpy as np

import bench
import oracle.moe_oracle as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layer_flops_match_the_oracle_count():
    for T, H, I, E, k in ((4096, 2048, 512, 256, 8), (64, 256, 128, 16, 2), (1, 2048, 512, 256, 8)):
        assert bench.layer_flops(T, H, I, E, k) == om.layer_flops(T, H, I, E, k)
    # 57,671,680 flop per token at the full shape: router 2HE, 8 routed + 1 shared SwiGLU experts
    assert bench.layer_flops(1, 2048, 512, 256, 8) == 57_671_680


def test_gate_up_flops_count_real_rows_only():
    # (T*k routed + T shared rows) x 2 x H x 2I
    assert bench.gateup_flops(4096, 2048, 512, 8) == (4096 * 9) * 2 * 2048 * 1024


def test_weight_bytes():
    assert bench.q4_bytes(512, 2048) == om.q4_bytes(512, 2048)
    assert bench.PER_EXPERT_BYTES == 1_769_472
    # one layer: 256 routed + 1 shared expert + the bf16 router matrix
    assert 257 * bench.PER_EXPERT_BYTES + 256 * 2048 * 2 == 455_802_880


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

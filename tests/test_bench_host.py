"""Host-side logic of bench.py (no GPU): the roofline each workload is held
against, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("name,bound", [("c1_gemm_bias_softmax_f32", "mfma"), ("c2_gemm_layernorm", "mfma"),
                                        ("c3_gemm_residual_rmsnorm", "mfma"), ("c4_b2b_mlp_relu", "hbm"),
                                        ("c5_b2b_attention", "mfma")])
def test_roofline_bound_follows_arithmetic_intensity(name, bound):
    w = gen.workload(name)
    b, unit, peak, achieved, intensity, ridge = bench.roofline_of(w, 1.0)
    assert b == bound
    assert (intensity < ridge) == (bound == "hbm")
    if bound == "hbm":
        assert unit == "GB/s" and peak == bench.HBM_GBPS
        assert achieved == pytest.approx(bench.bytes_of(w) / 1e-3 / 1e9)
    else:
        assert unit == "TFLOP/s"
        assert achieved == pytest.approx(bench.flops_of(w) / 1e-3 / 1e12)


def test_algorithmic_counts():
    w = gen.workload("c2_gemm_layernorm")
    assert bench.flops_of(w) == 2.0 * 8192 * 4096 * 4096
    # A, B, gamma, beta read once (bf16) + the bf16 output written once
    assert bench.bytes_of(w) == 2 * (8192 * 4096 + 4096 * 4096 + 4096 + 4096 + 8192 * 4096)
    # the second output X of a pre-norm block adds one bf16 [M, N] write
    w3 = gen.workload("c3_gemm_residual_rmsnorm")
    assert bench.bytes_of(w3, store_x=True) - bench.bytes_of(w3) == 2 * 16384 * 4096
    # an argmax writes an index and a maximum per row instead of the [M, N] output
    assert bench.bytes_of(w, argmax=True) == bench.bytes_of(w) - 2 * 8192 * 4096 + 8 * 8192
    w5 = gen.workload("c5_b2b_attention")
    assert bench.flops_of(w5) == 2.0 * 512 * 1024 * (64 * 1024 + 1024 * 64)
    # causal: row m of a square problem sees m + 1 keys
    assert bench.flops_of(w5, causal=True) == 2.0 * 512 * (1024 * 1025 // 2) * (64 + 64)
    assert bench.visible_pairs(3, 5) == 3 + 4 + 5 and bench.visible_pairs(5, 3) == 0 + 0 + 1 + 2 + 3


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("flags", [["--workload", "c4_b2b_mlp_relu", "--b-nk"],
                                   ["--workload", "c4_b2b_mlp_relu", "--argmax"],
                                   ["--workload", "c3_gemm_residual_rmsnorm", "--topk", "4"],
                                   ["--topk", "9"]])
def test_flags_outside_their_workloads_exit_with_message(flags):
    # rejected before any device work, so this runs without a GPU
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + flags, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "applies to" in r.stderr, r.stderr[-500:]

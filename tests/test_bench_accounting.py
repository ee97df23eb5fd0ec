"""The algorithmic counts behind bench.py's figures, checked on the CPU against
hand arithmetic and brute-force enumeration (no GPU, no library calls)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rdt_inputs import get_config  # noqa: E402


def test_gate_up_bytes_of_the_gqa_workload():
    """gqa: 512 tokens x top-2 = 1024 routed rows over 8 experts, D 1024,
    F 2816, bf16. Every expert used: 8 gate + 8 up matrices of 2816 x 1024,
    the 1024 rows read (1024 wide) and their SwiGLU outputs written (2816
    wide), 2 bytes each."""
    cfg = get_config("gqa")
    counts = [np.array([128] * 8)]
    weights = 8 * 2 * 2816 * 1024 * 2
    rows_in = 1024 * 1024 * 2
    rows_out = 1024 * 2816 * 2
    assert weights + rows_in + rows_out == 100_139_008
    assert bench.gate_up_bytes(cfg, counts, 2) == 100_139_008
    # an expert without rows streams no weights; averaging over loops
    skew = [np.array([256, 256, 0, 128, 128, 128, 64, 64]), np.array([128] * 8)]
    one_idle = 7 * 2 * 2816 * 1024 * 2 + rows_in + rows_out
    assert bench.gate_up_bytes(cfg, skew, 2) == (one_idle + 100_139_008) / 2


def test_attention_flops_match_pair_enumeration():
    """Causal attention FLOPs per token: every (query, key <= query) pair costs
    q.k and p.v, 2 * d multiply-adds per head; enumerate the pairs of one
    sequence and divide by its length."""
    cfg = get_config("gqa")
    S, H, d = cfg["seq"], cfg["n_heads"], cfg["head_dim"]
    pairs = sum(i + 1 for i in range(S))
    per_token = pairs * H * 2 * d * 2 / S
    assert abs(bench.flops_per_token_loop(cfg)["attention"] - per_token) < 1e-6 * per_token


def test_dense_and_expert_flops_of_the_gqa_workload():
    """QKV: 1024 x (16 + 2 * 4) * 64 weights; output projection 1024 x 1024;
    router 8 x 1024; experts: top-2 x (gate + up + down) of 1024 x 2816, two
    FLOPs per multiply-add."""
    f = bench.flops_per_token_loop(get_config("gqa"))
    assert f["qkv"] == 2 * 1024 * 1536
    assert f["out_proj"] == 2 * 1024 * 1024
    assert f["router"] == 2 * 1024 * 8
    assert f["experts"] == 2 * 3 * 2 * 1024 * 2816


def test_gate_up_kernel_label_follows_rows_per_expert():
    assert bench.gate_up_kernel(get_config("gqa")) == "k_grouped_gemm<bf16,160,128,0,2,4>"      # 128 rows
    # 1024 rows, 72 row tiles x 11 column tiles of 256x256: under four rounds of 256
    assert bench.gate_up_kernel(get_config("mla")) == "k_grouped_gemm<bf16,192,128,0,2,4>"
    # 1024 rows, 320 row tiles x 8 column tiles
    assert bench.gate_up_kernel(get_config("wide_moe")) == "k_grouped_gemm<bf16,256,256,0,2,8>"
    assert bench.gate_up_kernel(get_config("gqa_small")) == "k_grouped_gemm<bf16,64,64,0,3,4>"  # 40 rows
    assert bench.gate_up_kernel(get_config("tiny")) == "k_grouped_gemm<f32,128,128,0,2,4>"


def test_depth_attention_bytes_closed_form():
    """Per token: query and output (2 * Hd * dd) plus the keys and values of
    loops 0..t, (t + 1) on average (T + 1) / 2 over the T loops."""
    cfg = get_config("dreamer")
    N, T = cfg["batch"] * cfg["seq"], cfg["T"]
    Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
    per_loop = [N * (2 * Hd * dd + (t + 1) * 2 * KVd * dd) * 2 for t in range(T)]
    assert abs(bench.depth_attention_bytes(cfg, 2) - sum(per_loop) / T) < 1e-6 * sum(per_loop)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_wide_moe_kernel_accounting():
    """wide_moe: 8192 tokens, D 2048, 64 experts top-8 + 1 shared, F 1024, T 16,
    bf16, every expert receiving 1024 rows in every loop.
    gate/up: 4 * D * F FLOPs for each of the 8192 * 8 routed and 8192 shared rows;
    router: per token h, e, a read (3 * 4 * D), n2 written (2 * D), 8 indices,
    gates and slots (12 * 8) and a gap (4), plus the 64 x 2048 router weights;
    combine: per token h, e, a (12 * D), nine bf16 expert rows (9 * 2 * D),
    routing entries (12 * 8), h' (4 * D) and, except after the last loop, the
    next RMSNorm output (2 * D)."""
    cfg = get_config("wide_moe")
    counts = [np.full(64, 1024)] * 16
    assert bench.gate_up_flops(cfg, counts) == 4 * 2048 * 1024 * (65536 + 8192)
    assert bench.down_flops(cfg, counts) == 2 * 2048 * 1024 * (65536 + 8192)
    assert bench.router_bytes(cfg, counts, 2) == 8192 * (24576 + 4096 + 96 + 4) + 64 * 2048 * 2
    per = 24576 + 9 * 2 * 2048 + 96 + 8192
    assert bench.combine_bytes(cfg, counts, 2, 1) == 8192 * (15 * (per + 4096) + per) / 16
    assert bench.ksplit_of(cfg) == 1 and bench.ksplit_of(get_config("gqa")) == 2

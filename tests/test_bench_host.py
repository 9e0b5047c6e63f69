"""Host-side pieces of the benchmark: the steady-state split, the attention-path
label, the QK-gain weight sets and the hi | lo overhead count."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from ttt_inputs import get  # noqa: E402


def test_steady_start():
    # chunk index ceil(k/b) is the first whose window is full; 2.7B at 8K has none
    assert bench.steady_start(get("2.7b_128k")) == 8192
    assert bench.steady_start(get("2.7b_32k")) == 8192
    assert bench.steady_start(get("2.7b_8k")) is None
    assert bench.steady_start(get("1.3b_b4096")) == 8192
    assert bench.steady_start(get("tiny")) == 256
    assert bench.steady_start(get("tiny").with_(window=300)) == 384


def test_attention_path_thresholds():
    cfg = get("2.7b_128k")
    # B = 1.01 g sqrt(80) log2(e) = 13.03 g: fp16 bounded up to 14.5, bf16 bounded up to 48
    assert bench.attention_path(cfg, None) == {"fp16 bounded softmax": 32}
    assert bench.attention_path(cfg, bench.qk_gains(cfg, 2.0)) == {"bf16 bounded softmax": 32}
    assert bench.attention_path(cfg, bench.qk_gains(cfg, 4.0)) == {"bf16 online max": 32}
    assert bench.attention_path(get("tiny"), None) == {"fp32 online max": 2}


def test_qk_gains_are_bf16_and_hit_the_product():
    cfg = get("2.7b_8k")
    g = bench.qk_gains(cfg, 2.0)
    q, k = g["l0.q_norm"], g["l5.k_norm"]
    assert np.all(g["l3.attn_norm"] == 1.0) and np.all(g["final_norm"] == 1.0)
    bits = q.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)          # exactly representable in bf16
    assert abs(float(q[0] * k[0]) - 2.0) < 2e-3


def test_overhead_flops_counts_the_doubled_fast_reduction():
    cfg = get("2.7b_128k")
    ov = bench.overhead_flops(cfg, cfg.seq_len)
    d, F, nu, T = cfg.d_model, cfg.d_ff, cfg.n_update, cfg.seq_len
    assert ov["gemm_gate_up_swiglu"] + ov["gemm_down_residual"] == 6 * T * nu * d * F
    assert bench.overhead_flops(get("tiny"), 2048) == {}


def test_host_info_fields():
    hi = bench.host_info()
    assert hi["logical_cores"] >= 1
    assert "cpu_model" in hi and "physical_cores" in hi

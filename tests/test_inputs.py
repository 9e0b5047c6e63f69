"""Checks of the seeded input generators (CPU only)."""
import math

import numpy as np
import torch

from ttt_inputs import get, make_weights_np, make_tokens, tensor_specs
from ttt_inputs.weights import draw_np, draw_torch, round_bf16_np
from ttt_inputs.tokens import zipf_span_tokens


def test_numpy_and_torch_draws_are_bit_identical():
    for tid, shape, bf16 in [(0, (1000, 37), False), (7, (4096,), True), (1_000_001, (333, 65), True)]:
        a = draw_np(3, tid, shape, 0.02, bf16)
        b = draw_torch(3, tid, shape, 0.02, bf16, "cpu").to(torch.float32).numpy()
        assert np.array_equal(a, b)


def test_draw_moments():
    a = draw_np(0, 5, (1 << 20,), 0.02, False).astype(np.float64)
    assert abs(a.mean()) < 1e-4
    assert abs(a.std() - 0.02) < 1e-4
    assert np.max(np.abs(a)) <= 0.02 * math.sqrt(3 * 4) + 1e-6    # Irwin-Hall(4) support


def test_bf16_rounding_matches_torch():
    x = np.random.Generator(np.random.PCG64(0)).standard_normal(100000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16_np(x), ref)


def test_weight_layout_tiny():
    cfg = get("tiny")
    w = make_weights_np(cfg)
    names = [s[0] for s in tensor_specs(cfg)]
    assert set(w) == set(names)
    assert w["tok_emb"].shape == (256, 64) and w["fast0.w_down"].shape == (64, 256)
    assert np.all(w["l0.q_norm"] == 1.0)


def test_zipf_span_tokens():
    x, spans = zipf_span_tokens(20001, seed=1)
    assert x.min() >= 0 and x.max() < 128256
    covered = sum(ln for _, ln in spans)
    assert 0.05 * 20001 <= covered <= 0.05 * 20001 + 256
    for (d, ln), (d2, _) in zip(spans, spans[1:]):
        assert d + ln <= d2
    for d, ln in spans:
        assert 16 <= ln <= 256
    # every copied span occurs earlier in the stream
    for d, ln in spans[:20]:
        seg = x[d:d + ln]
        hay = x[:d]
        found = any(np.array_equal(hay[s:s + ln], seg) for s in range(0, d - ln + 1))
        assert found


def test_markov_tokens_deterministic():
    cfg = get("tiny")
    a = make_tokens(cfg, seed=1)
    b = make_tokens(cfg, seed=1)
    assert len(a) == cfg.seq_len + 1 and np.array_equal(a, b)
    assert a.max() < 256


def test_random_gains_distinct_and_bf16_exact():
    from ttt_inputs import TTTConfig, random_gains, round_bf16_np
    cfg = TTTConfig("g", 3, 256, 4, 64, 512, 1024, 600, 256, 128, 2, 0.5, "bf16")
    g = random_gains(cfg, 1, qk_range=(0.8, 1.05))
    assert len(g) == 3 * 4 + 1
    vals = [tuple(v[:4]) for v in g.values()]
    assert len(set(vals)) == len(vals)
    for k, v in g.items():
        lo, hi = (0.8, 1.05) if k.endswith(("q_norm", "k_norm")) else (0.5, 1.5)
        assert lo - 1e-2 <= v.min() and v.max() <= hi + 1e-2 and np.std(v) > 0.05 * (hi - lo)
        assert np.array_equal(v, round_bf16_np(v))
    g2 = random_gains(cfg, 1, qk_range=(0.8, 1.05))
    assert all(np.array_equal(g[k], g2[k]) for k in g)

"""GPU path against the oracle with non-unit gains on every norm.

Every RMSNorm of the model carries a learned gain (the block norms before
attention and before the MLPs, the final norm, and the per-head QK-norm): the
notes (section 6) count them among the frozen parameters phi.  The other GPU
tests use the unit gains of the workload generator, which cannot tell a gain
applied at the wrong index, a dropped gain or two norms' gains swapped.  Here
each gain vector is a distinct seeded draw in [0.5, 1.5] (bf16-exact), and the
GPU path is compared with the oracle on the same values, element by element,
covering the forward norms, the RMSNorm backward of the back-propagated blocks
(n_update >= 2), the frozen-prefix pass over several groups and a batch.

Tolerances as in the other parity tests: per-token loss |d| <= 1e-4 (fp32) and
<= 2e-2 (bf16); final fast weights rel-L2 <= 1e-5 / 1e-2; their change
dW = W_N - W_0 rel-L2 <= 1e-3 / 5e-2.
"""
import numpy as np
import pytest
import torch

from ttt_inputs import TTTConfig, get, make_tokens, make_weights_np, make_weights_torch, random_gains

from gpu_util import compare, fast_init, gpu_session, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mid(hd, dtype="bf16", T=600, n_update=2, L=3, eta=0.5, V=1024, k=256, b=128):
    H = 4
    F = {16: 192, 64: 512, 80: 704, 96: 768, 128: 1024}[hd]
    return TTTConfig(f"gains{hd}_{dtype}", L, H * hd, H, hd, F, V, T, k, b, n_update, eta, dtype, init_std=0.02)


def rand_tokens(n, vocab, seed):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=n).astype(np.int32)


def with_gains(cfg, seed, qk_range=None):
    g = random_gains(cfg, seed, qk_range=qk_range)
    return make_weights_torch(cfg, "cuda", gains=g), make_weights_np(cfg, gains=g), g


def check(cfg, gl, gf, ol, of, wn, tag):
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, wn), tag)
    if cfg.dtype == "fp32":
        assert dl <= 1e-4 and wr <= 1e-5 and dwr <= 1e-3
    else:
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


def test_tiny_fp32_gains():
    cfg = get("tiny")
    say("case: tiny fp32 with random gains")
    wt, wn, _ = with_gains(cfg, 1)
    tok = make_tokens(cfg, seed=1)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, _ = run_oracle(cfg, tok, weights_np=wn)
    check(cfg, gl, gf, ol, of, wn, "tiny gains")


def test_mid_fp32_gains_two_updated_blocks():
    cfg = mid(64, dtype="fp32", T=450, n_update=2)
    say("case: mid fp32 hd=64 n_u=2 random gains")
    wt, wn, _ = with_gains(cfg, 2)
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, 31)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, _ = run_oracle(cfg, tok, weights_np=wn)
    check(cfg, gl, gf, ol, of, wn, "mid fp32 gains")


@pytest.mark.parametrize("hd,qk", [(80, "small"), (64, "wide"), (96, "small"), (128, "small")])
def test_mid_bf16_gains(hd, qk):
    """qk "small": q/k gains in [0.8, 1.05], whose score bound keeps the attention
    forward in fp16; "wide": q/k gains in [0.5, 1.5] as well, which moves it to bf16."""
    cfg = mid(hd, T=600, n_update=2)
    say(f"case: mid bf16 hd={hd} n_u=2 random gains, qk {qk}")
    wt, wn, _ = with_gains(cfg, 3 + hd, qk_range=(0.8, 1.05) if qk == "small" else None)
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, 40 + hd)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, _ = run_oracle(cfg, tok, weights_np=wn)
    check(cfg, gl, gf, ol, of, wn, f"mid{hd} bf16 gains {qk}")


def test_frozen_prefix_groups_with_gains():
    """T past the largest group (16384 tokens): the frozen blocks run ahead over groups."""
    T = 16384 + 300
    cfg = mid(64, T=T, L=3, n_update=2, V=512, k=256, b=256)
    say(f"case: frozen prefix groups bf16 T={T} random gains")
    wt, wn, _ = with_gains(cfg, 7, qk_range=(0.8, 1.05))
    tok = rand_tokens(T + 1, cfg.vocab, 21)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, _ = run_oracle(cfg, tok, weights_np=wn)
    check(cfg, gl, gf, ol, of, wn, "groups gains")


def test_batch_with_gains():
    from oracle.ttt_oracle import Oracle
    from test_lm_prefill_amd import Session
    cfg = mid(64, T=384, n_update=2)
    B = 2
    say(f"case: batch B={B} bf16 random gains")
    wt, wn, _ = with_gains(cfg, 9)
    tok = np.random.Generator(np.random.PCG64(50)).integers(0, cfg.vocab, size=(B, cfg.seq_len + 1)).astype(np.int32)
    sess = Session(cfg, wt, max_tokens=cfg.seq_len, n_seq=B)
    l, f = sess.prefill(torch.from_numpy(tok).cuda(), want_fast=True)
    torch.cuda.synchronize()
    gl = l.double().cpu().numpy()
    gf = [[x.double().cpu().numpy() for x in fs] for fs in f]
    sess.close()
    for s in range(B):
        ol, W = Oracle(cfg, wn).prefill(tok[s])
        check(cfg, gl[s], gf[s], ol, [x for ws in W for x in ws], wn, f"batch gains seq {s}")

"""Batched independent sequences (one handle, n_seq = B) on the GPU.

Each sequence of the batch has its own fast weights and window; the frozen-
weight products run once over all B chunks.  Every sequence is compared with
the oracle run on that sequence alone (the usual tolerances); sequences are
independent (permuting the batch permutes every result bit for bit); graph
replay equals launch by launch; and each sequence matches a one-sequence
handle closely (the frozen products may split their reductions differently at
the larger row count, so only up to rounding).
"""
import numpy as np
import pytest
import torch

from ttt_inputs import TTTConfig, make_weights_np, make_weights_torch

from gpu_util import compare, fast_init, say

pytestmark = pytest.mark.gpu

TTT_NO_UPDATE, TTT_NO_GRAPH = 1, 2


def cfg_b(dtype="bf16", hd=64, T=600, L=3, n_update=2, k=256, b=128, V=1024, eta=0.5):
    H = 4
    F = {64: 512, 80: 704, 96: 768}[hd]
    return TTTConfig(f"batch{hd}_{dtype}", L, H * hd, H, hd, F, V, T, k, b, n_update, eta, dtype, init_std=0.02)


def batch_tokens(B, n, vocab, seed):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=(B, n)).astype(np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(sess, tok, flags=0):
    l, f = sess.prefill(torch.from_numpy(tok).cuda(), flags=flags, want_fast=True)
    torch.cuda.synchronize()
    return l.double().cpu().numpy(), [[x.double().cpu().numpy() for x in fs] for fs in f]


@pytest.mark.parametrize("dtype,hd,T,B", [("bf16", 64, 600, 3), ("bf16", 80, 512, 2), ("bf16", 96, 700, 2), ("fp32", 64, 450, 2)])
def test_batch_each_sequence_matches_oracle(dtype, hd, T, B):
    from oracle.ttt_oracle import Oracle
    from test_lm_prefill_amd import Session
    cfg = cfg_b(dtype=dtype, hd=hd, T=T)
    say(f"case: batch {dtype} hd={hd} T={T} B={B}")
    w = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    tok = batch_tokens(B, T + 1, cfg.vocab, seed=40 + hd + B)
    sess = Session(cfg, w, max_tokens=T, n_seq=B)
    gl, gf = _run(sess, tok)
    sess.close()
    tol = 1e-4 if dtype == "fp32" else 2e-2
    for s in range(B):
        ol, W = Oracle(cfg, wn).prefill(tok[s])
        of = [x for ws in W for x in ws]
        dl, wr, dwr = compare(cfg, gl[s], gf[s], ol, of, fast_init(cfg, wn), f"batch seq {s}")
        assert dl <= tol
        assert wr <= (1e-5 if dtype == "fp32" else 1e-2)
        assert dwr <= (1e-3 if dtype == "fp32" else 5e-2)


def test_batch_over_several_groups():
    # two sequences of 8892 tokens in 256-token chunks: the frozen-prefix pass takes groups of
    # at most 8192 tokens per sequence (at most 16384 rows over both), so each sequence spans a
    # whole group and a ragged one, and every chunk picks its rows from its own sequence's part
    # of the group
    from oracle.ttt_oracle import Oracle
    from test_lm_prefill_amd import Session
    T, B = 8192 + 700, 2
    cfg = cfg_b(dtype="fp32", hd=64, T=T, b=256, V=512)
    say(f"case: batch over groups fp32 T={T} B={B} b=256")
    w = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    tok = batch_tokens(B, T + 1, cfg.vocab, seed=91)
    sess = Session(cfg, w, max_tokens=T, n_seq=B)
    gl, gf = _run(sess, tok)
    sess.close()
    for s in range(B):
        ol, W = Oracle(cfg, wn).prefill(tok[s])
        of = [x for ws in W for x in ws]
        dl, wr, dwr = compare(cfg, gl[s], gf[s], ol, of, fast_init(cfg, wn), f"batch groups seq {s}")
        assert dl <= 1e-4
        assert wr <= 1e-5
        assert dwr <= 1e-3


def test_batch_invariants():
    from test_lm_prefill_amd import Session
    cfg = cfg_b(T=520)
    B = 3
    say("case: batch invariants bf16 B=3 T=520")
    w = make_weights_torch(cfg, "cuda")
    tok = batch_tokens(B, cfg.seq_len + 1, cfg.vocab, seed=77)
    sess = Session(cfg, w, max_tokens=cfg.seq_len, n_seq=B)
    l1, f1 = _run(sess, tok)
    l2, f2 = _run(sess, tok, flags=TTT_NO_GRAPH)
    assert np.array_equal(l1, l2)
    assert all(np.array_equal(a, b) for fa, fb in zip(f1, f2) for a, b in zip(fa, fb))
    perm = [2, 0, 1]
    lp, fp = _run(sess, np.ascontiguousarray(tok[perm]))
    for i, s in enumerate(perm):
        assert np.array_equal(lp[i], l1[s])
        assert all(np.array_equal(a, b) for a, b in zip(fp[i], f1[s]))
    l0, _ = _run(sess, tok, flags=TTT_NO_UPDATE)
    assert np.array_equal(l0[:, :cfg.chunk], l1[:, :cfg.chunk])   # chunk 0 precedes every update
    sess.close()
    one = Session(cfg, w, max_tokens=cfg.seq_len, n_seq=1)
    for s in range(B):
        ls, fs = one.prefill(torch.from_numpy(tok[s]).cuda(), want_fast=True)
        torch.cuda.synchronize()
        assert float(np.max(np.abs(ls.double().cpu().numpy() - l1[s]))) <= 2e-3
        num = sum(float(np.sum((a.double().cpu().numpy() - b) ** 2)) for a, b in zip(fs, f1[s]))
        den = sum(float(np.sum(b ** 2)) for b in f1[s])
        assert np.sqrt(num / den) <= 1e-4
    one.close()


def test_batch_rejects_decode():
    from test_lm_prefill_amd import Session
    from test_lm_prefill_amd.ttt import TTTError
    cfg = cfg_b(T=256)
    w = make_weights_torch(cfg, "cuda")
    sess = Session(cfg, w, max_tokens=300, n_seq=2)
    sess.prefill(torch.from_numpy(batch_tokens(2, 257, cfg.vocab, seed=1)).cuda(), want_fast=False)
    with pytest.raises(TTTError):
        sess.decode(4)
    sess.close()

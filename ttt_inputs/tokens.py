"""Seeded synthetic token streams (host side, numpy PCG64).

The pages measure on Books and DCLM text through the Llama-3 tokenizer; neither
is available, so these streams stand in for them at the pages' lengths and
vocabulary size.  No corpus content is reproduced.

* ``markov2``: an order-2 Markov chain over a small alphabet.  The law of the
  next symbol after context (a, c) mixes a global Zipf(1.5) law over a seeded
  permutation of the alphabet with a context-specific Dirichlet(0.1) draw, so a
  learner that adapts to the document can lower its loss.
* ``zipf_span``: i.i.d. Zipf(1.1) ranks over the vocabulary mapped to ids by a
  seeded permutation, then spans of 16..256 tokens copied from earlier in the
  same stream (sources may lie beyond the attention window) until about 5 % of
  the positions are copies.

This module holds no arithmetic of the method itself.
"""
import numpy as np


def _zipf_probs(n, s):
    r = np.arange(1, n + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def markov2_tokens(n_tokens, seed=1, vocab=256, zipf_s=1.5, alpha=0.1, mix=0.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(vocab)
    glob = np.empty(vocab)
    glob[perm] = _zipf_probs(vocab, zipf_s)
    g = rng.gamma(alpha, size=(vocab * vocab, vocab))
    g /= g.sum(axis=1, keepdims=True)
    table = mix * glob[None, :] + (1.0 - mix) * g
    cdf = np.cumsum(table, axis=1)
    cdf[:, -1] = 1.0
    x = np.empty(n_tokens, dtype=np.int64)
    x[:2] = rng.integers(0, vocab, size=min(2, n_tokens))[:n_tokens]
    u = rng.random(n_tokens)
    for t in range(2, n_tokens):
        row = cdf[x[t - 2] * vocab + x[t - 1]]
        x[t] = min(int(np.searchsorted(row, u[t], side="right")), vocab - 1)
    return x.astype(np.int32)


def zipf_span_tokens(n_tokens, seed=1, vocab=128256, zipf_s=1.1, copy_frac=0.05,
                     span_min=16, span_max=256):
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(vocab)
    cdf = np.cumsum(_zipf_probs(vocab, zipf_s))
    cdf[-1] = 1.0
    ranks = np.searchsorted(cdf, rng.random(n_tokens), side="right")
    x = perm[np.minimum(ranks, vocab - 1)].astype(np.int64)
    # choose non-overlapping destination spans until ~copy_frac of positions are copies
    target = int(copy_frac * n_tokens)
    taken = np.zeros(n_tokens, dtype=bool)
    spans = []
    covered, attempts = 0, 0
    while covered < target and attempts < 100000:
        attempts += 1
        ln = int(rng.integers(span_min, span_max + 1))
        if 2 * ln > n_tokens:
            break
        dst = int(rng.integers(ln, n_tokens - ln + 1))
        if taken[dst:dst + ln].any():
            continue
        taken[dst:dst + ln] = True
        spans.append((dst, ln))
        covered += ln
    for dst, ln in sorted(spans):
        src = int(rng.integers(0, dst - ln + 1))
        x[dst:dst + ln] = x[src:src + ln]
    return x.astype(np.int32), sorted(spans)


def make_tokens(cfg, seed=1, n_tokens=None):
    """T+1 ids for a workload (or n_tokens ids when given)."""
    n = cfg.seq_len + 1 if n_tokens is None else n_tokens
    if cfg.tokens == "markov2":
        return markov2_tokens(n, seed=seed, vocab=cfg.vocab)
    return zipf_span_tokens(n, seed=seed, vocab=cfg.vocab)[0]

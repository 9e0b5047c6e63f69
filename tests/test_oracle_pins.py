"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the passage of the pages (or the mathematical fact) it holds
the oracle to.  Torch library routines and finite differences serve as the
independent side; nothing here re-types the oracle's own formulas.
"""
import math

import numpy as np
import pytest
import torch

from oracle.ttt_oracle import Oracle, sgd_step
from ttt_inputs import TTTConfig, make_weights_np, make_tokens
import torch_ref

torch.set_num_threads(min(8, torch.get_num_threads()))


def micro(**kw):
    base = dict(name="micro", n_layers=2, d_model=16, n_heads=2, head_dim=8, d_ff=32, vocab=32,
                seq_len=32, window=12, chunk=8, n_update=2, eta=0.5, dtype="fp32", init_std=0.3,
                tokens="zipf_span")
    base.update(kw)
    return TTTConfig(**base)


def rand_gains(cfg, w, seed=5):
    """Non-unit norm gains so that their placement is exercised."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(w)
    for k, v in w.items():
        if k.endswith("norm"):
            out[k] = (1.0 + 0.2 * rng.standard_normal(v.shape)).astype(np.float32)
    return out


def rand_tokens(n, vocab, seed=3):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=n).astype(np.int32)


# ----------------------------------------------------------------------------- Pin 1
@pytest.mark.parametrize("n_u", [1, 2])
@pytest.mark.parametrize("chunk_idx", [0, 2])
def test_pin1_finite_differences(n_u, chunk_idx):
    """Hand-written gradient of A_i(W) (notes section 5, Eq. 9) vs central
    differences, with the attention state of earlier chunks held fixed
    (Alg. 1 step 3.4 differentiates at W_{i-1} only)."""
    cfg = micro(n_update=n_u)
    w = rand_gains(cfg, make_weights_np(cfg, seed=11))
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab)
    orc = Oracle(cfg, w)
    _, _, trace = orc.prefill(tok, return_trace=True)
    tr = trace[chunk_idx]
    W, cache, s0, n = tr["W_before"], tr["cache"], tr["s0"], tr["n"]
    if chunk_idx > 0:
        assert len(cache[-1]["pos"]) > 0   # state is populated
    _, saved, _ = orc.chunk_forward(W, cache, tok[s0:s0 + n], tok[s0 + 1:s0 + n + 1], s0)
    G = orc.chunk_grad(W, saved)
    h = 1e-5
    num, ana = [], []
    for u in range(n_u):
        for t in range(3):
            flat = W[u][t].reshape(-1)
            for j in range(flat.size):
                old = flat[j]
                flat[j] = old + h
                fp = orc.chunk_loss(W, cache, tok, s0, n)
                flat[j] = old - h
                fm = orc.chunk_loss(W, cache, tok, s0, n)
                flat[j] = old
                num.append((fp - fm) / (2 * h))
                ana.append(G[u][t].reshape(-1)[j])
    num, ana = np.array(num), np.array(ana)
    rel = np.linalg.norm(num - ana) / np.linalg.norm(ana)
    assert rel < 1e-6, rel


def test_pin1_ragged_last_chunk_finite_differences():
    """A short last chunk (T = 29, b = 8: the last chunk has n = 5 positions): the
    update's gradient is that of the mean loss over the chunk's own n positions
    (notes section 5, Eq. 9 averages over the chunk's targets; the pages leave a
    partial chunk open, and the plain reading is the mean over the targets it has).
    Central differences of numpy's mean over the n losses, with the window state of
    the earlier chunks held fixed, against the oracle's hand-written gradient; an
    oracle that divided by b instead of n would be off by n/b."""
    cfg = micro(n_update=2, seq_len=29)
    w = rand_gains(cfg, make_weights_np(cfg, seed=23))
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=24)
    orc = Oracle(cfg, w)
    _, _, trace = orc.prefill(tok, return_trace=True)
    tr = trace[-1]
    W, cache, s0, n = tr["W_before"], tr["cache"], tr["s0"], tr["n"]
    assert n == 5 and s0 == 24 and len(cache[-1]["pos"]) > 0
    _, saved, _ = orc.chunk_forward(W, cache, tok[s0:s0 + n], tok[s0 + 1:s0 + n + 1], s0)
    G = orc.chunk_grad(W, saved)

    def mean_loss():
        l_chunk, _, _ = orc.chunk_forward(W, cache, tok[s0:s0 + n], tok[s0 + 1:s0 + n + 1], s0)
        return float(np.mean(l_chunk))

    h = 1e-5
    num, ana = [], []
    for u in range(cfg.n_update):
        for t in range(3):
            flat = W[u][t].reshape(-1)
            for j in range(flat.size):
                old = flat[j]
                flat[j] = old + h
                fp = mean_loss()
                flat[j] = old - h
                fm = mean_loss()
                flat[j] = old
                num.append((fp - fm) / (2 * h))
                ana.append(G[u][t].reshape(-1)[j])
    num, ana = np.array(num), np.array(ana)
    rel = np.linalg.norm(num - ana) / np.linalg.norm(ana)
    assert rel < 1e-6, rel
    # the update the prefill applied is eta times that gradient
    _, WN = orc.prefill(tok)
    for ws, w0, g in zip(WN, W, G):
        for x, y, gg in zip(ws, w0, g):
            np.testing.assert_allclose(x, y - cfg.eta * gg, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- Pin 2 / 3
def _static_losses_torch(cfg, w, tok, mask):
    fast = torch_ref.fast_tensors(torch_ref.fast_from_weights(cfg, w))
    with torch.no_grad():
        return torch_ref.forward_losses(cfg, w, tok, fast, mask=mask).numpy()


@pytest.mark.parametrize("k,b", [(12, 8), (8, 8), (20, 4)])
def test_pin2_eta0_is_static_sliding_window(k, b):
    """eta = 0: the chunked recurrence with its bounded state equals one
    whole-sequence forward under the band mask p-k < j <= p (notes section 5:
    the window covers the chunk; Eq. 1 right side)."""
    cfg = micro(window=k, chunk=b, seq_len=40)
    w = rand_gains(cfg, make_weights_np(cfg, seed=12))
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=4)
    got, _ = Oracle(cfg, w).prefill(tok, eta=0.0)
    ref = _static_losses_torch(cfg, w, tok, "band")
    assert np.max(np.abs(got - ref)) < 1e-10


def test_pin2_tiny_workload_eta0():
    from ttt_inputs import get
    cfg = get("tiny")
    w = make_weights_np(cfg, seed=0)
    tok = make_tokens(cfg, seed=1)
    got, _ = Oracle(cfg, w).prefill(tok, no_update=True)
    ref = _static_losses_torch(cfg, w, tok, "band")
    assert np.max(np.abs(got - ref)) < 1e-10


def test_pin3_full_window_is_causal_attention():
    """k >= T: sliding-window attention is full causal attention."""
    cfg = micro(window=64, chunk=8, seq_len=40)
    w = rand_gains(cfg, make_weights_np(cfg, seed=13))
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=6)
    got, _ = Oracle(cfg, w).prefill(tok, eta=0.0)
    ref = _static_losses_torch(cfg, w, tok, "causal")
    assert np.max(np.abs(got - ref)) < 1e-10


# ----------------------------------------------------------------------------- Pin 4
def test_pin4_causality():
    """A token is predicted before it is used (notes section 2.2, last
    paragraph): later tokens change neither earlier losses nor the weights
    produced by earlier chunks."""
    cfg = micro()
    w = make_weights_np(cfg, seed=14)
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=7)
    orc = Oracle(cfg, w)
    base, _, tr = orc.prefill(tok, return_trace=True)
    for cut in [5, 8, 17, 24]:
        t2 = tok.copy()
        t2[cut + 1:] = (t2[cut + 1:] + 7) % cfg.vocab
        got, _, tr2 = orc.prefill(t2, return_trace=True)
        assert np.array_equal(got[:cut], base[:cut])          # positions < cut predict x_{<=cut}
        # chunk i's labels end at x_{(i+1)b}: chunks whose labels are all <= cut keep W_{i+1}
        i_done = (cut // cfg.chunk)
        for i in range(1, i_done + 1):
            for a, b2 in zip(tr[i]["W_before"], tr2[i]["W_before"]):
                for x, y in zip(a, b2):
                    assert np.array_equal(x, y)
        assert not np.array_equal(got, base)


# ----------------------------------------------------------------------------- Pin 5
class _UpdateFirst(Oracle):
    """Planted mistake: trains on the chunk before recording its losses."""

    def prefill(self, tokens, eta=None, no_update=False, W_init=None, return_trace=False):
        c = self.cfg
        eta = c.eta if eta is None else eta
        T = len(tokens) - 1
        W = self.init_fast()
        cache = self.empty_cache()
        losses = np.zeros(T)
        for s0 in range(0, T, c.chunk):
            n = min(c.chunk, T - s0)
            _, saved, _ = self.chunk_forward(W, cache, tokens[s0:s0 + n], tokens[s0 + 1:s0 + n + 1], s0)
            G = self.chunk_grad(W, saved)
            W = [[sgd_step(x, g, eta) for x, g in zip(ws, gs)] for ws, gs in zip(W, G)]
            l_chunk, _, cache = self.chunk_forward(W, cache, tokens[s0:s0 + n], tokens[s0 + 1:s0 + n + 1], s0)
            losses[s0:s0 + n] = l_chunk
        return losses, W


def _update_after_predict_holds(cls, cfg, w, tok):
    b = cfg.chunk
    l0, _ = cls(cfg, w).prefill(tok, eta=0.0)
    l1, _ = cls(cfg, w).prefill(tok, eta=cfg.eta)
    chunk0_same = np.array_equal(l0[:b], l1[:b])
    later_differ = not np.array_equal(l0[b:], l1[b:])
    return chunk0_same and later_differ


def test_pin5_update_after_predict():
    """Losses are recorded before the update (Alg. 1 step 3.3 before 3.5):
    chunk 0 cannot depend on eta, later chunks must; an oracle that trains
    first fails the same check."""
    cfg = micro()
    w = make_weights_np(cfg, seed=15)
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=8)
    assert _update_after_predict_holds(Oracle, cfg, w, tok)
    assert not _update_after_predict_holds(_UpdateFirst, cfg, w, tok)


# ----------------------------------------------------------------------------- Pin 6
@pytest.mark.parametrize("hd,d,k", [(64, 256, 64), (80, 320, 256), (96, 384, 64), (16, 64, 256)])
def test_pin6_one_chunk_matches_autograd(hd, d, k):
    """b = T: the update lands after every scored token (notes section 5, the
    b-equals-sequence boundary case), so losses are the static ones and
    W_1 = W_0 - eta * grad A(W_0) with grad from torch autograd."""
    F_ = {64: 704, 80: 864, 96: 1040, 16: 176}[hd]
    T = 256
    cfg = TTTConfig("pin6", 3, d, d // hd, hd, F_, 1024, T, k, T, 2, 0.05, "fp32", init_std=0.05)
    w = rand_gains(cfg, make_weights_np(cfg, seed=16))
    tok = rand_tokens(T + 1, cfg.vocab, seed=9)
    losses, W1 = Oracle(cfg, w).prefill(tok)
    fast = torch_ref.fast_tensors(torch_ref.fast_from_weights(cfg, w), requires_grad=True)
    ref = torch_ref.forward_losses(cfg, w, tok, fast, mask="band")
    assert np.max(np.abs(losses - ref.detach().numpy())) < 1e-10
    ref.mean().backward()
    num = den = 0.0
    for u in range(cfg.n_update):
        for t in range(3):
            w1_ref = fast[u][t].detach().numpy() - cfg.eta * fast[u][t].grad.numpy()
            dw_ref = w1_ref - fast[u][t].detach().numpy()
            dw = W1[u][t] - fast[u][t].detach().numpy()
            num += np.sum((dw - dw_ref) ** 2)
            den += np.sum(dw_ref ** 2)
    assert math.sqrt(num / den) < 1e-9


@pytest.mark.parametrize("T,b", [(100, 128), (77, 256)])
def test_pin6_partial_single_chunk_matches_autograd(T, b):
    """One chunk shorter than b (T not a multiple of 64): W_1 = W_0 - eta * grad of
    the mean over its T losses, with grad from torch autograd of torch's mean over
    the T cross-entropies (notes section 5, Eq. 9; reading: a partial chunk is
    averaged over its own positions)."""
    hd, d = 64, 256
    cfg = TTTConfig("pin6r", 3, d, d // hd, hd, 704, 1024, T, 64, b, 2, 0.05, "fp32", init_std=0.05)
    w = rand_gains(cfg, make_weights_np(cfg, seed=26))
    tok = rand_tokens(T + 1, cfg.vocab, seed=27)
    losses, W1 = Oracle(cfg, w).prefill(tok)
    fast = torch_ref.fast_tensors(torch_ref.fast_from_weights(cfg, w), requires_grad=True)
    ref = torch_ref.forward_losses(cfg, w, tok, fast, mask="band")
    assert ref.shape[0] == T
    assert np.max(np.abs(losses - ref.detach().numpy())) < 1e-10
    ref.mean().backward()
    num = den = 0.0
    for u in range(cfg.n_update):
        for t in range(3):
            dw_ref = -cfg.eta * fast[u][t].grad.numpy()
            dw = W1[u][t] - fast[u][t].detach().numpy()
            num += np.sum((dw - dw_ref) ** 2)
            den += np.sum(dw_ref ** 2)
    assert math.sqrt(num / den) < 1e-9


# ----------------------------------------------------------------------------- Pin 7
def test_pin7_prefix_consistency():
    """Running a prefix of m chunks reproduces the first m chunks of the full
    run exactly (Alg. 1 is causal in chunk order)."""
    cfg = micro()
    w = make_weights_np(cfg, seed=17)
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=10)
    orc = Oracle(cfg, w)
    full, WN, tr = orc.prefill(tok, return_trace=True)
    for m in [1, 2, 3]:
        pre, Wm = orc.prefill(tok[:m * cfg.chunk + 1])
        assert np.array_equal(pre, full[:m * cfg.chunk])
        if m < len(tr):
            for a, b2 in zip(Wm, tr[m]["W_before"]):
                for x, y in zip(a, b2):
                    assert np.array_equal(x, y)


# ----------------------------------------------------------------------------- Pin 8
@pytest.mark.parametrize("cfgname", ["tiny", "vocab_wide"])
def test_pin8_initial_loss_closed_form(cfgname):
    """At random init the final RMSNorm makes |n|^2 = d, so logits are ~N(0, d sigma^2)
    and E[loss] ~ ln V + d sigma^2 / 2 (cross-entropy as in the notes, section 2.2)."""
    from ttt_inputs import get
    if cfgname == "tiny":
        cfg = get("tiny")
    else:
        cfg = TTTConfig("vw", 1, 64, 4, 16, 128, 128256, 256, 256, 256, 1, 0.01, "fp32")
    w = make_weights_np(cfg, seed=0)
    tok = make_tokens(cfg, seed=1)[: cfg.chunk + 1]
    losses, _ = Oracle(cfg, w).prefill(tok, no_update=True)
    s2 = cfg.d_model * cfg.init_std ** 2
    expect = math.log(cfg.vocab) + s2 / 2
    sigma = math.sqrt(s2) / math.sqrt(cfg.chunk)
    assert abs(losses.mean() - expect) < 4 * sigma + 2e-3, (losses.mean(), expect, sigma)


# ----------------------------------------------------------------------------- Pin 9
def test_pin9_quadratic_gd_closed_form():
    """Eq. (8) of the notes (section 4.2, Fig. 3: a=1, w*=1, w0=0): the SGD rule
    on A(w) = a (w - w*)^2 / 2 gives e_i = (1 - eta a)^i e_0."""
    a, ws = 1.0, 1.0
    for eta in [0.5, 0.25, 1.5, 1.9, 2.1]:
        w = np.array([0.0])
        for i in range(1, 30):
            w = sgd_step(w, a * (w - ws), eta)
            e = (1 - eta * a) ** i * (0.0 - ws)
            assert abs(w[0] - ws - e) <= 1e-12 * max(1.0, abs(e))
    # shrinks iff 0 < eta a < 2
    for eta, shrink in [(0.1, True), (1.99, True), (2.01, False)]:
        w = np.array([0.0])
        for _ in range(50):
            w = sgd_step(w, a * (w - ws), eta)
        assert (abs(w[0] - ws) < 1.0) == shrink


# ----------------------------------------------------------------------------- Pin 10
def test_pin10_per_token_updates():
    """b = 1 with the attention output switched off is the attention-free toy
    of the notes' section 3, Eq. (3): predict x_t from x_{t-1} with W_{t-1},
    then W_t = W_{t-1} - eta grad l_t."""
    cfg = micro(chunk=1, seq_len=12, n_update=2, eta=0.3)
    w = rand_gains(cfg, make_weights_np(cfg, seed=18))
    for l in range(cfg.n_layers):
        w[f"l{l}.wo"] = np.zeros_like(w[f"l{l}.wo"])
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=11)
    losses, WN = Oracle(cfg, w).prefill(tok)
    fast = torch_ref.fast_tensors(torch_ref.fast_from_weights(cfg, w))
    ref_losses = []
    for t in range(cfg.seq_len):
        params = [[x.detach().clone().requires_grad_(True) for x in ws] for ws in fast]
        lt = torch_ref.forward_losses(cfg, w, tok[t:t + 2], params, mask="causal")[0]
        lt.backward()
        ref_losses.append(lt.item())
        fast = [[x.detach() - cfg.eta * x.grad for x in ws] for ws in params]
    assert np.max(np.abs(losses - np.array(ref_losses))) < 1e-12
    for a, b2 in zip(WN, fast):
        for x, y in zip(a, b2):
            assert np.max(np.abs(x - y.numpy())) < 1e-12


# ----------------------------------------------------------------------------- Pin 11
def test_pin11_zero_fast_branch():
    """A zero fast MLP with eta = 0 adds exactly nothing: the model equals the
    same network without fast weights (the static branch alone, notes section 6)."""
    cfg = micro()
    w = make_weights_np(cfg, seed=19)
    for k in list(w):
        if k.startswith("fast"):
            w[k] = np.zeros_like(w[k])
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=12)
    a, _ = Oracle(cfg, w).prefill(tok, eta=0.0)
    cfg0 = cfg.with_(n_update=0)
    b2, _ = Oracle(cfg0, w).prefill(tok)
    assert np.array_equal(a, b2)


# ----------------------------------------------------------------------------- Pin 12
@pytest.mark.parametrize("T,k,b", [(40, 12, 8), (64, 16, 16), (33, 20, 4)])
def test_pin12_key_count(T, k, b):
    """Eq. (1) of the notes (section 2.1): the window attends sum_t min(t, k) pairs."""
    cfg = micro(seq_len=T, window=k, chunk=b)
    w = make_weights_np(cfg, seed=20)
    tok = rand_tokens(T + 1, cfg.vocab, seed=13)
    orc = Oracle(cfg, w)
    orc.prefill(tok, no_update=True)
    expect = cfg.n_layers * sum(min(t, k) for t in range(1, T + 1))
    assert orc.key_count == expect


# ----------------------------------------------------------------------------- Pin 13
def test_pin13_learnability_tiny():
    """Directional: on the Markov stream, inner updates lower the loss of late
    chunks (the method's premise, notes section 1)."""
    from ttt_inputs import get
    cfg = get("tiny")
    w = make_weights_np(cfg, seed=0)
    tok = make_tokens(cfg, seed=1)
    l_ttt, _ = Oracle(cfg, w).prefill(tok)
    l_static, _ = Oracle(cfg, w).prefill(tok, no_update=True)
    b = cfg.chunk
    late_ttt = l_ttt[-4 * b:].mean()
    late_static = l_static[-4 * b:].mean()
    assert np.array_equal(l_ttt[:b], l_static[:b])
    assert late_static - late_ttt > 0.01, (late_static, late_ttt)


# ----------------------------------------------------------------------------- ragged/empty
def test_ragged_last_chunk_and_empty():
    """A short last chunk is averaged over its own size (a reading: the pages
    leave partial chunks open); T = 0 returns nothing and W_init."""
    cfg = micro(seq_len=29)
    w = make_weights_np(cfg, seed=21)
    tok = rand_tokens(30, cfg.vocab, seed=14)
    orc = Oracle(cfg, w)
    losses, WN, tr = orc.prefill(tok, return_trace=True)
    assert len(losses) == 29 and tr[-1]["n"] == 5
    # the last update uses the mean over the 5 scored positions: compare with b=T' prefill
    last = tr[-1]
    _, saved, _ = orc.chunk_forward(last["W_before"], last["cache"], tok[24:29], tok[25:30], 24)
    G = orc.chunk_grad(last["W_before"], saved)
    for ws, w0, g in zip(WN, last["W_before"], G):
        for x, y, gg in zip(ws, w0, g):
            assert np.array_equal(x, y - cfg.eta * gg)
    l0, W0 = orc.prefill(tok[:1])
    assert len(l0) == 0
    for ws, u in zip(W0, range(cfg.n_update)):
        assert np.array_equal(ws[0], w[f"fast{u}.w_gate"].astype(np.float64))


# ----------------------------------------------------------------------------- Pin 14
def test_pin14_decode_eta0_is_greedy_generation():
    """Algorithm 3 with the inner step size zero is plain greedy generation with the
    frozen model: every generated id is the argmax of the next-token logits of the
    whole sequence so far (an independent torch forward over the prefix), and every
    step loss is that forward's cross-entropy of the generated id."""
    cfg = micro(eta=0.0, window=12, chunk=8)
    w = rand_gains(cfg, make_weights_np(cfg))
    prompt = rand_tokens(17, cfg.vocab, seed=21)       # 16 scored positions
    o = Oracle(cfg, w)
    _, ids, step_losses, margins, _ = o.decode(prompt, 20)
    fast = torch_ref.fast_tensors(torch_ref.fast_from_weights(cfg, w))
    seq = list(prompt)
    with torch.no_grad():
        for j in range(20):
            z = torch_ref.forward_losses(cfg, w, seq + [0], fast, mask="band", return_logits=True)[-1].numpy()
            assert margins[j] > 1e-9
            assert int(np.argmax(z)) == ids[j], j
            lse = np.log(np.sum(np.exp(z - z.max()))) + z.max()
            assert abs((lse - z[ids[j]]) - step_losses[j]) < 1e-10, j
            seq.append(int(ids[j]))


@pytest.mark.parametrize("greedy", [False, True])
def test_pin15_decode_updates_follow_algorithm1(greedy):
    """Algorithm 3's update after every b generated ids is Algorithm 1's chunk step
    on the generated sequence: with the prompt a whole number of chunks, decoding
    (forced or greedy) and then prefilling the prompt plus the generated ids give
    the same fast weights and the same per-position losses; a shorter decode is a
    prefix of a longer one."""
    cfg = micro(eta=0.5, window=12, chunk=8)
    w = rand_gains(cfg, make_weights_np(cfg))
    prompt = rand_tokens(17, cfg.vocab, seed=22)
    n = 24                                              # three decode chunks
    forced = None if greedy else rand_tokens(n, cfg.vocab, seed=23)
    o = Oracle(cfg, w)
    pre, ids, step_losses, _, W = o.decode(prompt, n, forced=forced)
    if forced is not None:
        assert np.array_equal(ids, forced)
    full = np.concatenate([prompt, ids]).astype(np.int64)
    l_full, W_full = Oracle(cfg, w).prefill(full)
    np.testing.assert_allclose(l_full[:16], pre, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_full[16:], step_losses, rtol=0, atol=1e-10)
    for a, b in zip([x for ws in W for x in ws], [x for ws in W_full for x in ws]):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # the decode updates did something, and the first chunk's ids precede them
    _, ids0, sl0, _, W0 = Oracle(cfg, w).decode(prompt, n, forced=forced, no_update=True)
    assert np.max(np.abs(step_losses[8:] - sl0[8:])) > 1e-4
    if greedy:
        _, ids_pre, sl_pre, _, _ = Oracle(cfg, w).decode(prompt, 11)
        assert np.array_equal(ids_pre, ids[:11])
        np.testing.assert_allclose(sl_pre, step_losses[:11], rtol=0, atol=1e-12)

"""GPU path (libttt through its C ABI) against the CPU oracle, element by element.

Tolerances: per-token loss |d| <= 1e-4 (fp32 workloads) and <= 2e-2 (bf16),
final fast weights rel-L2 <= 1e-2 (bf16).  The change of the fast weights,
dW = W_N - W_0, is compared too, because W_N alone is dominated by W_0.
"""
import numpy as np
import pytest
import torch

from ttt_inputs import TTTConfig, get, make_tokens

from gpu_util import compare, fast_init, gpu_session, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

TTT_NO_UPDATE, TTT_NO_GRAPH = 1, 2


def mid(hd, dtype="bf16", T=600, n_update=2, L=3, eta=0.5, std=0.02, V=1024, k=256, b=128):
    H = 4
    d = H * hd
    F = {16: 192, 32: 384, 64: 512, 80: 704, 96: 768, 128: 1024}[hd]
    return TTTConfig(f"mid{hd}_{dtype}", L, d, H, hd, F, V, T, k, b, n_update, eta, dtype, init_std=std)


def rand_tokens(n, vocab, seed=3):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=n).astype(np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(0)


def test_weights_generated_on_device_match_host():
    from ttt_inputs import make_weights_np, make_weights_torch
    cfg = mid(64)
    wt = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    for k in ["tok_emb", "l1.wq", "fast0.w_down", "l2.w_up"]:
        assert np.array_equal(wt[k].float().cpu().numpy(), wn[k]), k


def test_tiny_fp32_full_sequence():
    cfg = get("tiny")
    say("case: tiny fp32 T=2048")
    tok = make_tokens(cfg, seed=1)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), "tiny")
    assert dl <= 1e-4
    assert wr <= 1e-5
    assert dwr <= 1e-3


@pytest.mark.parametrize("hd", [16, 32, 64, 80, 96, 128])
def test_mid_bf16_ragged(hd):
    cfg = mid(hd)
    say(f"case: mid hd={hd} bf16 T={cfg.seq_len} b={cfg.chunk} k={cfg.window}")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=hd)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"mid{hd}")
    assert dl <= 2e-2
    assert wr <= 1e-2
    assert dwr <= 5e-2


def test_mid_fp32_hd64():
    cfg = mid(64, dtype="fp32")
    say("case: mid hd=64 fp32")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=7)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), "mid64 fp32")
    assert dl <= 1e-4
    assert dwr <= 1e-3


@pytest.mark.parametrize("head_scale", [1, 12])
def test_no_update_equals_eta0_and_bitwise_invariants(head_scale):
    # head_scale 12: the first 128 head rows scaled so that the weights fail the single-pass
    # head's bound, and the head runs its two-pass form
    from ttt_inputs import make_weights_np, make_weights_torch
    cfg = mid(80, T=512)
    say(f"case: invariants hd=80 bf16 T=512 head rows x{head_scale}")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=11)
    wt = make_weights_torch(cfg, "cuda")
    wt["lm_head"][:128] *= head_scale
    wn = make_weights_np(cfg)
    wn["lm_head"][:128] = wt["lm_head"][:128].float().cpu().numpy()
    assert head_bound_test(cfg, wn) == (head_scale == 1)
    sess, w = gpu_session(cfg, weights=wt)
    sess0, _ = gpu_session(cfg.with_(eta=0.0), weights=w)
    l_upd, f1 = run_gpu(sess, tok)
    l_upd2, f2 = run_gpu(sess, tok)
    # determinism: two runs bit-identical
    assert np.array_equal(l_upd, l_upd2)
    assert all(np.array_equal(a, b) for a, b in zip(f1, f2))
    # graph replay == launch-by-launch
    l_ng, f_ng = run_gpu(sess, tok, flags=TTT_NO_GRAPH)
    assert np.array_equal(l_upd, l_ng)
    assert all(np.array_equal(a, b) for a, b in zip(f1, f_ng))
    # NO_UPDATE == eta = 0
    l_nu, _ = run_gpu(sess, tok, flags=TTT_NO_UPDATE)
    l_e0, _ = run_gpu(sess0, tok)
    assert np.array_equal(l_nu, l_e0)
    # update-after-predict: chunk 0 independent of eta, later chunks not
    b = cfg.chunk
    assert np.array_equal(l_upd[:b], l_nu[:b])
    assert not np.array_equal(l_upd[b:], l_nu[b:])
    # causality: perturbing tokens after position cut leaves losses[:cut] unchanged
    cut = 300
    t2 = tok.copy()
    t2[cut + 1:] = (t2[cut + 1:] + 5) % cfg.vocab
    l_c, _ = run_gpu(sess, t2)
    assert np.array_equal(l_c[:cut], l_upd[:cut])
    # prefix consistency: a run over the first m chunks reproduces them
    for m in [1, 2, 3]:
        l_p, _ = run_gpu(sess, tok[:m * b + 1])
        assert np.array_equal(l_p, l_upd[:m * b]), m


def test_empty_and_single_chunk():
    cfg = mid(64, T=256)
    sess, w = gpu_session(cfg)
    l0, f0 = run_gpu(sess, rand_tokens(1, cfg.vocab))
    assert len(l0) == 0
    from ttt_inputs import make_weights_np
    wn = make_weights_np(cfg)
    for a, b in zip(f0, fast_init(cfg, wn)):
        assert np.array_equal(a, b)
    tok = rand_tokens(cfg.chunk + 1, cfg.vocab, seed=5)
    gl, gf = run_gpu(sess, tok)
    ol, of, wn = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, wn), "one chunk")
    assert dl <= 2e-2 and dwr <= 5e-2


@pytest.mark.parametrize("hd", [64, 80, 96, 128])
def test_long_window_split_attention(hd):
    """A window of 1024 with 128-token chunks: the attention passes split the
    key range over several work-groups and the ring wraps (T > k + b)."""
    cfg = mid(hd, T=1700, k=1024, b=128, L=2)
    say(f"case: long window hd={hd} T={cfg.seq_len} k={cfg.window} b={cfg.chunk}")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=100 + hd)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"longwin{hd}")
    assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


def _with_gains(cfg, gq, gk):
    """Weights of cfg with QK-norm gains replaced (bf16-exact values)."""
    from ttt_inputs import make_weights_np, make_weights_torch
    from ttt_inputs.weights import round_bf16_np
    wt = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    for l in range(cfg.n_layers):
        for nm, g in ((f"l{l}.q_norm", gq(l)), (f"l{l}.k_norm", gk(l))):
            g = round_bf16_np(np.asarray(g, dtype=np.float32))
            wn[nm] = g
            wt[nm] = torch.from_numpy(g).to(device="cuda", dtype=wt[nm].dtype)
    return wt, wn


@pytest.mark.parametrize("case", ["varied", "large"])
def test_qk_gains_score_bound(case):
    """The forward uses a fixed softmax offset derived from the QK-norm gains
    when that bound is small ("varied": gains in [0.5, 1.5]) and the running
    maximum otherwise ("large": one q gain of 8 puts the bound past its limit
    while the scores stay moderate, so bf16 keeps the usual tolerance)."""
    cfg = mid(64, T=700, k=256, b=128)
    rng = np.random.Generator(np.random.PCG64(11))
    if case == "varied":
        gq = lambda l: rng.uniform(0.5, 1.5, cfg.head_dim)
        gk = lambda l: rng.uniform(0.5, 1.5, cfg.head_dim)
    else:
        gq = lambda l: np.concatenate([[8.0], np.ones(cfg.head_dim - 1)])
        gk = lambda l: np.ones(cfg.head_dim)
    wt, wn = _with_gains(cfg, gq, gk)
    say(f"case: qk gains {case} T={cfg.seq_len}")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=77)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, _ = run_oracle(cfg, tok, weights_np=wn)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, wn), f"gains-{case}")
    assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


@pytest.mark.parametrize("dtype,n_update", [("bf16", 0), ("bf16", 2), ("fp32", 0)])
def test_window_covers_sequence(dtype, n_update):
    """Full causal attention: the window (and the ring, k + b rows) covers the
    whole sequence, so no key is ever evicted.  n_update = 0 is the plain
    Transformer timed as the full-attention baseline; with updates it is
    TTT over full attention."""
    T = 700
    cfg = mid(64, dtype=dtype, T=T, k=768, b=128, n_update=n_update)
    say(f"case: full window {dtype} n_update={n_update} T={T} k={cfg.window}")
    tok = rand_tokens(T + 1, cfg.vocab, seed=200 + n_update)
    sess, _ = gpu_session(cfg)
    flags = TTT_NO_UPDATE if n_update == 0 else 0
    gl, gf = run_gpu(sess, tok, flags=flags, want_fast=n_update > 0)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf if n_update else None, ol, of if n_update else None, fast_init(cfg, w),
                          f"fullwin {dtype} nu={n_update}")
    assert dl <= (1e-4 if dtype == "fp32" else 2e-2)
    if n_update:
        assert wr <= 1e-2 and dwr <= 5e-2


@pytest.mark.parametrize("n_update,L", [(1, 3), (4, 4)])
def test_n_update_extremes(n_update, L):
    """One updated block, and every block updated (the first block's attention
    is then back-propagated too only from blocks above it)."""
    cfg = mid(64, T=600, L=L, n_update=n_update)
    say(f"case: n_update={n_update} of L={L}")
    tok = rand_tokens(cfg.seq_len + 1, cfg.vocab, seed=300 + n_update)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"nu={n_update}/L={L}")
    assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


@pytest.mark.parametrize("dtype,k,b", [("bf16", 128, 128), ("fp32", 64, 64), ("bf16", 64, 64)])
def test_window_equal_to_chunk(dtype, k, b):
    """The smallest window the library accepts, k = b: a chunk's last query sees only
    its own chunk, its first query the whole previous chunk but one key, and the ring
    (k + b rows) holds exactly two chunks.  T is ragged."""
    T = 9 * b + 37
    cfg = mid(64, dtype=dtype, T=T, k=k, b=b)
    say(f"case: window = chunk {dtype} k={k} b={b} T={T}")
    tok = rand_tokens(T + 1, cfg.vocab, seed=400 + k)
    sess, _ = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"k=b={k} {dtype}")
    if dtype == "fp32":
        assert dl <= 1e-4 and wr <= 1e-5 and dwr <= 1e-3
    else:
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


def head_bound_test(cfg, w):
    """The library's create-time test for running the head's loss and gradient in one pass:
    every row's logits lie within 2 * 1.01 sqrt(d) max|g_final| max_v |W_v| of its label's
    logit, and that spread plus ln V stays at or below 126."""
    wn = float(np.max(np.linalg.norm(w["lm_head"].astype(np.float64), axis=1)))
    gm = float(np.max(np.abs(w["final_norm"])))
    return 2 * 1.01 * wn * gm * np.sqrt(cfg.d_model) + np.log(cfg.vocab) <= 126.0


@pytest.mark.parametrize("dtype,V,b,scale", [("bf16", 1040, 128, 8), ("fp32", 1008, 128, 8), ("bf16", 40016, 1024, 8),
                                             ("bf16", 1040, 128, 12), ("fp32", 1008, 128, 16),
                                             ("bf16", 40016, 1024, 12)])
def test_ragged_vocab(dtype, V, b, scale):
    """A vocabulary that is a multiple of 16 but not of 128: the head's last column tile
    and its cross-entropy partials are ragged; at b = 1024 the head backward streams the
    vocabulary in slabs of 32768 columns, so the second slab is ragged too.  The first 128
    head rows are scaled (the oracle takes the scaled values as stored): their logits dominate
    every row's softmax, so a partial slot of them lost or overwritten would move the
    losses by O(1).  At scale 8 the weights pass the single-pass head's bound; at 12 and 16
    they do not, and the head computes the losses first and the softmax after."""
    from ttt_inputs import make_weights_np, make_weights_torch
    T = 2 * b + 52
    cfg = mid(64, dtype=dtype, T=T, V=V, b=b, k=max(256, b))
    say(f"case: ragged vocab {dtype} V={V} b={b} T={T} head rows x{scale}")
    tok = rand_tokens(cfg.seq_len + 1, V, seed=500 + V)
    tok[::7] = V - 1  # the last vocabulary rows are labels too
    wt = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    wt["lm_head"][:128] *= scale
    # the oracle takes the stored (rounded, for bf16) values
    wn["lm_head"][:128] = wt["lm_head"][:128].float().cpu().numpy()
    assert head_bound_test(cfg, wn) == (scale == 8)
    sess, _ = gpu_session(cfg, weights=wt)
    gl, gf = run_gpu(sess, tok)
    ol, of, w = run_oracle(cfg, tok, weights_np=wn)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"V={V} {dtype} x{scale}")
    if dtype == "fp32":
        assert dl <= 1e-4 and wr <= 1e-5 and dwr <= 1e-3
    else:
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


def wide_tiles(M, N):
    return -(-M // 256) * -(-N // 256)


@pytest.mark.parametrize("B,b", [(1, 1024), (2, 512)])
def test_grouped_gate_up_launch(B, b):
    """An updated block's static gate/up product (all sequences) and each sequence's fast
    one fill less than the GPU's 256 CUs with 256 x 256 tiles alone; with at least 200 such
    tiles together they run as one launch (d = 1024, 2F = 6656: 104 tiles for each of the
    static and the fast product at 1024 rows; B = 2 at b = 512: three products)."""
    from test_lm_prefill_amd import Session
    from ttt_inputs import make_weights_np, make_weights_torch
    T = 2 * b + 100
    cfg = TTTConfig("grouped_bf16", 2, 1024, 8, 128, 3328, 1024, T, b, b, 1, 0.5, "bf16", init_std=0.02)
    static = wide_tiles(B * b, 2 * cfg.d_ff)
    fast = B * wide_tiles(b, 2 * cfg.d_ff)
    assert static < 200 and fast // B < 200 and static + fast >= 200
    say(f"case: grouped gate/up B={B} b={b} T={T} ({static} + {fast} wide tiles)")
    w = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    toks = [rand_tokens(T + 1, cfg.vocab, seed=700 + s) for s in range(B)]
    sess = Session(cfg, w, max_tokens=T, n_seq=B)
    l, f = sess.prefill(torch.from_numpy(np.stack(toks)).cuda() if B > 1 else torch.from_numpy(toks[0]).cuda(),
                        want_fast=True)
    torch.cuda.synchronize()
    sess.close()
    for s in range(B):
        gl = (l[s] if B > 1 else l).double().cpu().numpy()
        gf = [x.double().cpu().numpy() for x in (f[s] if B > 1 else f)]
        ol, of, _ = run_oracle(cfg, toks[s], weights_np=wn)
        dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, wn), f"grouped B={B} seq {s}")
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2


def test_fp32_shapes_off_the_64_grid():
    """fp32 mode accepts d_model, d_ff and vocab that are multiples of 16 only: three heads
    of 16 (d = 48), d_ff = 208, V = 1008, T = 1 (one scored position) and a ragged T."""
    cfg = TTTConfig("odd_fp32", 2, 48, 3, 16, 208, 1008, 345, 128, 64, 1, 0.5, "fp32", init_std=0.05)
    say("case: fp32 d=48 F=208 V=1008")
    sess, _ = gpu_session(cfg)
    for T, seed in ((1, 601), (345, 602)):
        tok = rand_tokens(T + 1, cfg.vocab, seed=seed)
        gl, gf = run_gpu(sess, tok)
        ol, of, w = run_oracle(cfg, tok)
        dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, w), f"odd fp32 T={T}")
        assert len(gl) == T
        assert dl <= 1e-4 and wr <= 1e-5 and dwr <= 1e-3


# the largest frozen-prefix group the library forms for one sequence (it picks 8192 to
# 16384 rows from a time model of the frozen pass)
GROUP = 16384


@pytest.mark.parametrize("dtype,hd,T", [("fp32", 16, GROUP + 300), ("bf16", 64, GROUP + 300), ("bf16", 80, GROUP + 300)])
def test_frozen_prefix_over_several_groups(dtype, hd, T):
    # T spans at least two groups (the last one ragged), so the blocks below the
    # updated ones run ahead over each group and the chunks pick their rows from it
    cfg = mid(hd, dtype=dtype, T=T, L=3, n_update=2, V=512, k=256, b=256)
    say(f"case: frozen prefix over groups {dtype} hd={hd} T={T} L=3 n_u=2 b=256")
    tok = rand_tokens(T + 1, cfg.vocab, seed=21)
    sess, w = gpu_session(cfg)
    gl, gf = run_gpu(sess, tok)
    ol, of, wn = run_oracle(cfg, tok)
    dl, wr, dwr = compare(cfg, gl, gf, ol, of, fast_init(cfg, wn), f"groups {dtype}")
    if dtype == "fp32":
        assert dl <= 1e-4 and wr <= 1e-5 and dwr <= 1e-3
    else:
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2
    # the number of rows of the group a position falls in does not change its result:
    # shorter runs (one group of fewer rows; a second group of three chunks) reproduce the
    # long run's losses bit for bit.  A ragged last chunk of a few rows may take other
    # kernels in the updated blocks, so only the positions before it are compared there.
    b = cfg.chunk
    for n, m in [(20 * b + 17, 20 * b + 17), (GROUP // 2 + 3 * b, GROUP // 2 + 3 * b),
                 (GROUP // 2 + 3 * b + 5, GROUP // 2 + 3 * b)]:
        if n < T:
            l_p, _ = run_gpu(sess, tok[:n + 1])
            bad = np.nonzero(l_p[:m] != gl[:m])[0]
            assert bad.size == 0, (n, bad[:5])
    # with graph replay the next group's frozen-prefix pass runs on a second stream beside
    # the chunk steps; launched one by one, everything runs on one stream: same bits
    l_ng, f_ng = run_gpu(sess, tok, flags=TTT_NO_GRAPH)
    assert np.array_equal(l_ng, gl)
    assert all(np.array_equal(a, c) for a, c in zip(f_ng, gf))

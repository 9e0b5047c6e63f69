"""Algorithm 3 (generation with periodic updates) on the GPU against the oracle.

Forced ids (teacher forcing) make the bf16 comparison well defined: the step
losses within 2e-2 and the fast weights after the decode updates within the
prefill tolerances.  Greedy decoding is compared id by id in fp32, up to the
first step whose top-2 logit margin in the oracle is below 5e-5 (a near tie that
fp32 rounding may decide either way).  Bitwise invariants: graph replay equals
launch by launch; a greedy decode equals a forced decode of the ids it chose;
two decode calls equal one; after a decode, the fast weights equal those of a
prefill over the prompt plus the generated ids.
"""
import numpy as np
import pytest
import torch

from ttt_inputs import TTTConfig

from gpu_util import compare, fast_init, gpu_session, say

pytestmark = pytest.mark.gpu

TTT_NO_UPDATE, TTT_NO_GRAPH = 1, 2


def cfg_dec(dtype="bf16", hd=64, L=3, n_update=2, k=256, b=128, V=1024, eta=0.5):
    H = 4
    F = {64: 512, 80: 704, 96: 768, 128: 1024}[hd]
    return TTTConfig(f"dec{hd}_{dtype}", L, H * hd, H, hd, F, V, 2048, k, b, n_update, eta, dtype, init_std=0.02)


def rand_tokens(n, vocab, seed):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=n).astype(np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_decode(cfg, prompt, n, forced=None, w=None):
    from oracle.ttt_oracle import Oracle
    from ttt_inputs import make_weights_np
    w = make_weights_np(cfg) if w is None else w
    pre, ids, sl, margins, W = Oracle(cfg, w).decode(prompt, n, forced=forced)
    return pre, ids, sl, margins, [x for ws in W for x in ws], w


def _gpu_decode(sess, prompt, n, forced=None, flags=0):
    tok = torch.from_numpy(np.asarray(prompt, dtype=np.int32)).cuda()
    pre, _ = sess.prefill(tok, flags=flags, want_fast=False)
    f = torch.from_numpy(np.asarray(forced, dtype=np.int32)).cuda() if forced is not None else None
    ids, sl, fast = sess.decode(n, forced=f, flags=flags)
    torch.cuda.synchronize()
    return (pre.double().cpu().numpy(), ids.cpu().numpy(), sl.double().cpu().numpy(),
            [x.double().cpu().numpy() for x in fast] if fast is not None else None)


@pytest.mark.parametrize("hd,P", [(64, 256), (80, 200), (96, 300), (128, 384)])
def test_decode_forced_bf16(hd, P):
    """Prompt of P positions (a whole number of chunks, or not), then 300 forced
    steps: two decode updates and an open chunk at the end."""
    cfg = cfg_dec(hd=hd)
    n = 300
    prompt = rand_tokens(P + 1, cfg.vocab, seed=hd)
    forced = rand_tokens(n, cfg.vocab, seed=hd + 1)
    say(f"case: decode forced bf16 hd={hd} P={P} n={n}")
    sess, _ = gpu_session(cfg)
    gpre, gids, gsl, gf = _gpu_decode(sess, prompt, n, forced)
    opre, oids, osl, _, of, w = _oracle_decode(cfg, prompt, n, forced)
    assert np.array_equal(gids, forced)
    dl_pre = float(np.max(np.abs(gpre - opre)))
    dl, wr, dwr = compare(cfg, gsl, gf, osl, of, fast_init(cfg, w), f"decode forced hd={hd}")
    say(f"prefill max|dloss|={dl_pre:.3e}")
    assert dl_pre <= 2e-2 and dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2
    sess.close()


def test_decode_two_pass_head_bf16():
    """Head row 0 scaled by 13 (the oracle takes the stored value): the weights fail the
    single-pass head's bound, so each decode update's head runs the cross-entropy pass and
    then the softmax pass.  Forced steps against the oracle, and a greedy decode equal to
    a forced decode of the ids it chose, bit for bit."""
    from ttt_inputs import make_weights_np, make_weights_torch
    cfg = cfg_dec(hd=64)
    n, P = 300, 256
    wt = make_weights_torch(cfg, "cuda")
    wt["lm_head"][:1] *= 13
    wn = make_weights_np(cfg)
    wn["lm_head"][:1] = wt["lm_head"][:1].float().cpu().numpy()
    bound = 2 * 1.01 * np.max(np.linalg.norm(wn["lm_head"].astype(np.float64), axis=1)) * np.sqrt(cfg.d_model)
    assert bound + np.log(cfg.vocab) > 126.0
    prompt = rand_tokens(P + 1, cfg.vocab, seed=77)
    forced = rand_tokens(n, cfg.vocab, seed=78)
    say(f"case: decode forced bf16, two-pass head, P={P} n={n}")
    sess, _ = gpu_session(cfg, weights=wt)
    gpre, gids, gsl, gf = _gpu_decode(sess, prompt, n, forced)
    opre, oids, osl, _, of, w = _oracle_decode(cfg, prompt, n, forced, w=wn)
    dl_pre = float(np.max(np.abs(gpre - opre)))
    dl, wr, dwr = compare(cfg, gsl, gf, osl, of, fast_init(cfg, w), "decode forced, two-pass head")
    say(f"prefill max|dloss|={dl_pre:.3e}")
    assert dl_pre <= 2e-2 and dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2
    _, ids, sl, f = _gpu_decode(sess, prompt, n)
    _, ids3, sl3, f3 = _gpu_decode(sess, prompt, n, forced=ids)
    assert np.array_equal(sl, sl3) and all(np.array_equal(x, y) for x, y in zip(f, f3))
    sess.close()


def test_decode_greedy_fp32():
    cfg = cfg_dec(dtype="fp32", k=256, b=64)
    n, P = 160, 128
    prompt = rand_tokens(P + 1, cfg.vocab, seed=5)
    say(f"case: decode greedy fp32 P={P} n={n}")
    sess, _ = gpu_session(cfg)
    gpre, gids, gsl, gf = _gpu_decode(sess, prompt, n)
    opre, oids, osl, margins, of, w = _oracle_decode(cfg, prompt, n)
    tie = np.nonzero(margins < 5e-5)[0]
    upto = int(tie[0]) if len(tie) else n
    say(f"greedy ids compared over {upto} of {n} steps; smallest oracle margin {margins.min():.2e}")
    assert upto >= cfg.chunk + 8, "too few steps before a near tie to cover a decode update"
    assert np.array_equal(gids[:upto], oids[:upto])
    assert float(np.max(np.abs(gsl[:upto] - osl[:upto]))) <= 1e-4
    assert float(np.max(np.abs(gpre - opre))) <= 1e-4
    if upto == n:
        dl, wr, dwr = compare(cfg, gsl, gf, osl, of, fast_init(cfg, w), "decode greedy fp32")
        assert wr <= 1e-5 and dwr <= 1e-3
    sess.close()


def test_decode_bitwise_invariants():
    cfg = cfg_dec(hd=64)
    P, n = 256, 300
    prompt = rand_tokens(P + 1, cfg.vocab, seed=9)
    say("case: decode invariants bf16")
    sess, _ = gpu_session(cfg)
    _, ids, sl, f = _gpu_decode(sess, prompt, n)                      # greedy, graph replay
    _, ids2, sl2, f2 = _gpu_decode(sess, prompt, n, flags=TTT_NO_GRAPH)
    assert np.array_equal(ids, ids2) and np.array_equal(sl, sl2)
    assert all(np.array_equal(a, b) for a, b in zip(f, f2))
    _, ids3, sl3, f3 = _gpu_decode(sess, prompt, n, forced=ids)      # forced = the greedy choice
    assert np.array_equal(sl, sl3) and all(np.array_equal(a, b) for a, b in zip(f, f3))
    # two calls (the second continues an open chunk) equal one
    tok = torch.from_numpy(prompt).cuda()
    sess.prefill(tok, want_fast=False)
    ia, sa, _ = sess.decode(100)
    ib, sb, fb = sess.decode(n - 100)
    assert np.array_equal(np.concatenate([ia.cpu().numpy(), ib.cpu().numpy()]), ids)
    assert np.array_equal(np.concatenate([sa.cpu().numpy(), sb.cpu().numpy()]), sl.astype(np.float32))
    assert all(np.array_equal(a.double().cpu().numpy(), b) for a, b in zip(fb, f))
    # the decode updates are Algorithm 1's chunk steps on the generated sequence
    full = np.concatenate([prompt, ids]).astype(np.int32)
    n_pos = P + (n // cfg.chunk) * cfg.chunk               # the decoded chunks that were closed
    lp, fp = sess.prefill(torch.from_numpy(full[:n_pos + 1]).cuda(), want_fast=True)
    assert all(np.array_equal(a.double().cpu().numpy(), b) for a, b in zip(fp, f))
    # with no update the decode leaves the prefill's weights
    _, fpre = sess.prefill(tok, want_fast=True)
    _, _, f0 = sess.decode(n, flags=TTT_NO_UPDATE)
    assert all(torch.equal(a, b) for a, b in zip(f0, fpre))
    sess.close()


def test_decode_argument_checks():
    from test_lm_prefill_amd.ttt import TTTError
    cfg = cfg_dec(hd=64)
    sess, _ = gpu_session(cfg, max_tokens=300)
    with pytest.raises(TTTError):
        sess.decode(4)                                       # no prefill yet
    sess.prefill(torch.from_numpy(rand_tokens(257, cfg.vocab, seed=1)).cuda(), want_fast=False)
    with pytest.raises(TTTError):
        sess.decode(100)                                     # 256 + 100 > max_tokens
    ids, sl, _ = sess.decode(44)                             # exactly up to max_tokens
    assert ids.numel() == 44 and bool(torch.isfinite(sl).all())
    sess.close()

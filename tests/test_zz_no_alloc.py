"""ttt_prefill_noalloc (the entry point that allocates nothing) against ttt_prefill.

The two run the same kernels with the same split-K and key-range-split plans;
only the memory the partial results go to differs (a static device array of the
library instead of the handle's workspaces), so their results are compared bit
for bit, besides the usual oracle tolerances.  Two calls in a row, the second on
a shorter, ragged sequence, check that what the first call leaves in the shared
array does not leak into the second.  The shape uses split-K products (K up to
4F over 128 rows) and split attention (window 1024 over chunks of 128).
"""
import numpy as np
import pytest
import torch

from ttt_inputs import TTTConfig, make_weights_np, make_weights_torch

from gpu_util import compare, fast_init, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfg(T=1700):
    return TTTConfig("noalloc64", 2, 256, 4, 64, 512, 1024, T, 1024, 128, 2, 0.5, "bf16", init_std=0.02)


def _noalloc(sess, tok):
    from test_lm_prefill_amd import ttt
    T = tok.numel() - 1
    losses = torch.empty(T, dtype=torch.float32, device="cuda")
    fast = sess._fast_buffers(torch.device("cuda"))
    stream = torch.cuda.current_stream().cuda_stream
    ttt.ttt_prefill_noalloc(sess.handle, tok.data_ptr(), T, losses.data_ptr(), [t.data_ptr() for t in fast], 0,
                            stream)
    ttt.ttt_check_finite(sess.handle, stream)
    torch.cuda.synchronize()
    return losses.double().cpu().numpy(), [f.double().cpu().numpy() for f in fast]


def _regular(sess, tok):
    l, f = sess.prefill(tok, want_fast=True)
    torch.cuda.synchronize()
    return l.double().cpu().numpy(), [x.double().cpu().numpy() for x in f]


def test_noalloc_matches_prefill_on_two_calls():
    from test_lm_prefill_amd import Session
    cfg = _cfg()
    w = make_weights_torch(cfg, "cuda")
    wn = make_weights_np(cfg)
    sess = Session(cfg, w)
    rng = np.random.Generator(np.random.PCG64(61))
    tok_np = rng.integers(0, cfg.vocab, cfg.seq_len + 1).astype(np.int32)
    for T in (cfg.seq_len, 900 + 37):   # the second call shorter, with a ragged last chunk
        say(f"case: noalloc vs prefill T={T}")
        tok = torch.from_numpy(tok_np[:T + 1].copy()).cuda()
        nl, nf = _noalloc(sess, tok)
        rl, rf = _regular(sess, tok)
        assert np.array_equal(nl, rl)
        assert all(np.array_equal(a, b) for a, b in zip(nf, rf))
        ol, of, _ = run_oracle(cfg.with_(seq_len=T), tok_np[:T + 1], weights_np=wn)
        dl, wr, dwr = compare(cfg, nl, nf, ol, of, fast_init(cfg, wn), f"noalloc T={T}")
        assert dl <= 2e-2 and wr <= 1e-2 and dwr <= 5e-2
    # the regular call after them still matches its own earlier result
    tok = torch.from_numpy(tok_np.copy()).cuda()
    nl, _ = _noalloc(sess, tok)
    rl, _ = _regular(sess, tok)
    assert np.array_equal(nl, rl)
    sess.close()


def test_noalloc_rejects_what_does_not_fit():
    from test_lm_prefill_amd import Session, ttt
    # 8 * b * d = 8 * 4096 * 1024 floats of split-K partials exceed the 96 MiB of the array
    cfg = TTTConfig("noalloc_big", 1, 1024, 16, 64, 1024, 256, 4096, 4096, 4096, 1, 0.01, "bf16")
    sess = Session(cfg, make_weights_torch(cfg, "cuda"))
    tok = torch.zeros(cfg.seq_len + 1, dtype=torch.int32, device="cuda")
    losses = torch.empty(cfg.seq_len, dtype=torch.float32, device="cuda")
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_prefill_noalloc(sess.handle, tok.data_ptr(), cfg.seq_len, losses.data_ptr(), None, 0,
                                torch.cuda.current_stream().cuda_stream)
    assert e.value.status == ttt.TTT_EUNSUPPORTED and "scratch" in str(e.value)
    # kernel timing creates events, so it is refused
    sess.set_kernel_timing(True)
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_prefill_noalloc(sess.handle, tok.data_ptr(), 0, None, None, 0, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == ttt.TTT_EINVAL
    sess.close()

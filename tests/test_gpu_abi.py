"""The C ABI's status and statistics on the GPU.

TTT_ENONFINITE covers the inner update as well as the recorded losses
(Algorithm 1 of the notes: the losses of step 3.3 come before the gradient and
SGD step of 3.4-3.5, so a non-finite update can leave every recorded loss
finite).  The condition is forced from the host: one chunk, a final-norm gain
of 1e30 (the logits and losses stay finite, the gradient into the fast weights
is about 1e26) and eta = 1e20, so the SGD step overflows to infinity.  Every
kernel runs to its normal end; only the status reports it.
"""
import numpy as np
import pytest
import torch

from ttt_inputs import get, make_tokens, make_weights_torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _one_chunk(eta):
    from test_lm_prefill_amd import Session
    from test_lm_prefill_amd.ttt import TTTError, TTT_ENONFINITE
    cfg = get("tiny").with_(seq_len=128, eta=eta)
    w = make_weights_torch(cfg, "cuda")
    w["final_norm"] = torch.full_like(w["final_norm"], 1e30)
    tok = torch.from_numpy(make_tokens(get("tiny"), seed=1)[:cfg.seq_len + 1].copy()).cuda()
    sess = Session(cfg, w)
    losses, fast = sess.prefill(tok, want_fast=True, check=False)
    torch.cuda.synchronize()
    status = 0
    try:
        sess.prefill(tok, want_fast=False, check=True)
    except TTTError as e:
        status = e.status
    stats = sess.stats()
    sess.close()
    return losses.cpu().numpy(), [f.cpu().numpy() for f in fast], status, stats, TTT_ENONFINITE


def test_nonfinite_update_sets_the_status():
    say("case: one chunk, final-norm gain 1e30, eta 1e20")
    losses, fast, status, _, ENONFINITE = _one_chunk(1e20)
    assert np.all(np.isfinite(losses))
    assert any(not np.all(np.isfinite(f)) for f in fast)
    assert status == ENONFINITE


def test_finite_update_is_ok_and_stats():
    say("case: one chunk, final-norm gain 1e30, eta 1e-3")
    losses, fast, status, stats, _ = _one_chunk(1e-3)
    assert np.all(np.isfinite(losses)) and all(np.all(np.isfinite(f)) for f in fast)
    assert status == 0
    ms, chunks, launches = stats
    assert chunks == 1 and launches > 0 and ms > 0.0


def test_stats_time_of_last_prefill():
    from test_lm_prefill_amd import Session
    cfg = get("tiny")
    sess = Session(cfg, make_weights_torch(cfg, "cuda"))
    assert sess.stats()[0] == 0.0
    tok = torch.from_numpy(make_tokens(cfg, seed=1)).cuda()
    sess.prefill(tok, want_fast=False)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    sess.prefill(tok, want_fast=False, check=False)
    e1.record()
    torch.cuda.synchronize()
    ms, chunks, _ = sess.stats()
    sess.close()
    outer = e0.elapsed_time(e1)
    say(f"ms_last {ms:.3f} outer events {outer:.3f}")
    assert chunks == cfg.seq_len // cfg.chunk
    assert 0.0 < ms <= outer * 1.01 + 0.05

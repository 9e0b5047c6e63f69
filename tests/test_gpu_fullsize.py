"""Full-size workloads on the GPU against stored oracle results.

fp32 mode: the 125M workload (head dim 64) runs the fp32 path on the same
bf16-valued weights and must match every per-token loss of the whole
32768-token sequence to 1e-4.

For each workload the session is created exactly as the benchmark creates it
(the workload's own weights, max_tokens = its full sequence length, graph
replay), then:

* a prefix run over the first chunks the oracle ran (tests/golden/, written by
  make_golden.py from oracle/ and ttt_inputs/ only) is compared element by
  element: every per-token loss within 2e-2 (bf16), sampled entries of the
  final fast weights within rel-L2 1e-2 and of their change W_N - W_0 within
  rel-L2 5e-2;
* the full-length run must reproduce the prefix run's losses bit for bit on
  those chunks (a prefix cannot see later tokens) and every loss is finite.
"""
import os

import numpy as np
import pytest
import torch

from ttt_inputs import get, make_tokens, make_weights_torch

from gpu_util import say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAMES = ["125m", "760m", "1.3b_b256", "1.3b_b1024", "1.3b_b4096", "2.7b_8k", "2.7b_32k", "2.7b_128k"]


def _golden(name):
    p = os.path.join(GOLDEN, f"oracle_{name}.npz")
    if not os.path.exists(p):
        pytest.skip(f"no stored oracle result for {name}")
    return np.load(p)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sampled_rel(gf, g, n_t, key):
    num = den = 0.0
    for t in range(n_t):
        idx = g[f"idx_{t}"]
        gv = gf[t].reshape(-1)[torch.as_tensor(idx, device=gf[t].device)].double().cpu().numpy()
        ref = g[f"{key}_{t}"] if key == "w" else g[f"w_{t}"] - g[f"w0_{t}"]
        got = gv if key == "w" else gv - g[f"w0_{t}"]
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    return np.sqrt(num / den)


def test_fullsize_fp32_whole_sequence_125m():
    from test_lm_prefill_amd import Session
    g = _golden("125m")
    cfg = get("125m")
    assert int(g["T"]) == cfg.seq_len
    say(f"case: 125m fp32 T={cfg.seq_len}")
    tok = torch.from_numpy(make_tokens(cfg, seed=1)).cuda()
    w = {k: v.float() for k, v in make_weights_torch(cfg, "cuda", seed=0).items()}
    sess = Session(cfg.with_(dtype="fp32"), w, max_tokens=cfg.seq_len)
    try:
        lp, fp = sess.prefill(tok, want_fast=True)
        torch.cuda.synchronize()
        dl = float(np.max(np.abs(lp.double().cpu().numpy() - g["losses"].astype(np.float64))))
        n_t = 3 * cfg.n_update
        wr = _sampled_rel(fp, g, n_t, "w")
        dwr = _sampled_rel(fp, g, n_t, "dw")
        say(f"[125m fp32] max|dloss|={dl:.3e} W rel-L2={wr:.3e} dW rel-L2={dwr:.3e}")
        assert dl <= 1e-4
        assert wr <= 1e-5
        assert dwr <= 1e-3
    finally:
        sess.close()
        del w
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_against_oracle_prefix(name):
    from test_lm_prefill_amd import Session
    g = _golden(name)
    cfg = get(name)
    Tp = int(g["T"])
    say(f"case: {name} prefix T={Tp} of {cfg.seq_len}")
    tok_np = make_tokens(cfg, seed=1)
    w = make_weights_torch(cfg, "cuda", seed=0)
    sess = Session(cfg, w, max_tokens=cfg.seq_len)
    try:
        tok = torch.from_numpy(tok_np).cuda()
        lp, fp = sess.prefill(tok[: Tp + 1].contiguous(), want_fast=True)
        torch.cuda.synchronize()
        gl = lp.double().cpu().numpy()
        dl = float(np.max(np.abs(gl - g["losses"].astype(np.float64))))
        n_t = 3 * cfg.n_update
        wr = _sampled_rel(fp, g, n_t, "w")
        dwr = _sampled_rel(fp, g, n_t, "dw")
        say(f"[{name}] prefix: max|dloss|={dl:.3e} W rel-L2={wr:.3e} dW rel-L2={dwr:.3e} "
            f"mean loss gpu {gl.mean():.4f} oracle {g['losses'].mean():.4f}")
        del fp
        assert dl <= 2e-2
        assert wr <= 1e-2
        assert dwr <= 5e-2
        if Tp < cfg.seq_len:
            lf, _ = sess.prefill(tok, want_fast=False)
            torch.cuda.synchronize()
            lf = lf.cpu().numpy()
            say(f"[{name}] full T={cfg.seq_len}: mean loss {lf.mean():.4f}")
            assert np.all(np.isfinite(lf))
            assert np.array_equal(lf[:Tp], lp.cpu().numpy())
    finally:
        sess.close()
        del w
        torch.cuda.empty_cache()

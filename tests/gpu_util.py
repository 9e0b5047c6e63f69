"""Helpers shared by the GPU tests: run the HIP path and the oracle on the same inputs."""
import sys

import numpy as np
import torch

from ttt_inputs import make_weights_np, make_weights_torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_session(cfg, seed=0, max_tokens=None, weights=None):
    from test_lm_prefill_amd import Session
    w = weights if weights is not None else make_weights_torch(cfg, "cuda", seed=seed)
    return Session(cfg, w, max_tokens=max_tokens), w


def run_gpu(sess, tokens_np, flags=0, want_fast=True):
    tok = torch.as_tensor(np.asarray(tokens_np, dtype=np.int32)).cuda()
    losses, fast = sess.prefill(tok, flags=flags, want_fast=want_fast)
    torch.cuda.synchronize()
    out_fast = None
    if fast is not None:
        out_fast = [f.cpu().numpy().astype(np.float64) for f in fast]
    return losses.cpu().numpy().astype(np.float64), out_fast


def run_oracle(cfg, tokens_np, seed=0, no_update=False, weights_np=None):
    from oracle.ttt_oracle import Oracle
    w = weights_np if weights_np is not None else make_weights_np(cfg, seed=seed)
    losses, W = Oracle(cfg, w).prefill(np.asarray(tokens_np), no_update=no_update)
    flat = [x for ws in W for x in ws]
    return losses, flat, w


def fast_init(cfg, w_np):
    return [w_np[f"fast{u}.{n}"].astype(np.float64) for u in range(cfg.n_update)
            for n in ("w_gate", "w_up", "w_down")]


def rel_l2(a_list, b_list):
    num = sum(float(np.sum((a - b) ** 2)) for a, b in zip(a_list, b_list))
    den = sum(float(np.sum(b ** 2)) for b in b_list)
    return np.sqrt(num / den) if den > 0 else np.sqrt(num)


def compare(cfg, gl, gf, ol, of, w0, tag=""):
    """Returns (max |dloss|, W_N rel-L2, dW rel-L2)."""
    dl = float(np.max(np.abs(gl - ol))) if len(ol) else 0.0
    wr = rel_l2(gf, of) if of else 0.0
    dg = [g - w for g, w in zip(gf, w0)] if of else []
    do = [o - w for o, w in zip(of, w0)] if of else []
    dwr = rel_l2(dg, do) if of else 0.0
    say(f"[{tag}] max|dloss|={dl:.3e}  W rel-L2={wr:.3e}  dW rel-L2={dwr:.3e}  "
        f"|dW|/|W0|={rel_l2(do, [0 * x for x in do]) / max(1e-30, rel_l2(w0, [0 * x for x in w0])) if of else 0:.3e}")
    return dl, wr, dwr

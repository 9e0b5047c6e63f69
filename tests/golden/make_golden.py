"""Writes the expected values the full-size GPU parity tests compare against.

Calls only the CPU oracle (oracle/) and the seeded input generators
(ttt_inputs/).  For each workload it runs Algorithm 1 of the reading notes
(section 7) on the first `chunks` chunks of the workload's own token stream
(the prefix the full-length run sees; a prefix run reproduces the first chunks
of the full run exactly) and stores:

  losses      float32 [chunks * b]   per-token losses of those chunks
  idx_<t>     int32   [S]            sampled flat indices of fast tensor t
  w_<t>       float64 [S]            W after `chunks` updates at those indices
  w0_<t>      float64 [S]            W_init at those indices

Usage: python tests/golden/make_golden.py [workload ...]

The script re-executes itself once with glibc's malloc told to keep freed
memory (no mmap for large blocks): the oracle allocates gigabyte temporaries
per chunk, and first-touch page faults would otherwise dominate its run time.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle.ttt_oracle import Oracle  # noqa: E402
from ttt_inputs import get, make_tokens, make_weights_np  # noqa: E402

# workload -> number of leading chunks the oracle runs (None = whole sequence).
# k/b + 2 chunks fill the window and wrap the key/value ring (R = k + b rows).
PLAN = {
    "125m": None,
    "760m": 10,
    "1.3b_b256": 34,
    "1.3b_b1024": 10,
    "1.3b_b4096": 4,
    "2.7b_8k": None,
    "2.7b_32k": 3,
    "2.7b_128k": 10,
}
SAMPLES = 1024


def fast_names(cfg):
    return [f"fast{u}.{n}" for u in range(cfg.n_update) for n in ("w_gate", "w_up", "w_down")]


def make(name, weights_cache):
    cfg = get(name)
    chunks = PLAN[name]
    T = cfg.seq_len if chunks is None else chunks * cfg.chunk
    key = (cfg.n_layers, cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_update)
    if key not in weights_cache:
        weights_cache.clear()
        t0 = time.time()
        weights_cache[key] = make_weights_np(cfg, seed=0)
        print(f"[{name}] weights in {time.time() - t0:.0f}s", flush=True)
    w = weights_cache[key]
    tok = make_tokens(cfg, seed=1)[: T + 1]
    t0 = time.time()
    def progress(s0, n):
        print(f"[{name}] chunk at {s0} done, {time.time() - t0:.0f}s", flush=True)

    losses, W = Oracle(cfg, w).prefill(tok, progress=progress)
    print(f"[{name}] oracle over {T} tokens in {time.time() - t0:.0f}s, mean loss {losses.mean():.4f}", flush=True)
    out = {"losses": losses.astype(np.float32), "T": np.int64(T), "chunk": np.int64(cfg.chunk)}
    rng = np.random.Generator(np.random.PCG64(7))
    flat_w = [x for ws in W for x in ws]
    for t, (nm, wn) in enumerate(zip(fast_names(cfg), flat_w)):
        idx = np.sort(rng.choice(wn.size, size=min(SAMPLES, wn.size), replace=False))
        out[f"idx_{t}"] = idx.astype(np.int32)
        out[f"w_{t}"] = wn.reshape(-1)[idx].astype(np.float64)
        out[f"w0_{t}"] = w[nm].reshape(-1)[idx].astype(np.float64)
    path = os.path.join(HERE, f"oracle_{name}.npz")
    np.savez_compressed(path, **out)
    print(f"[{name}] wrote {path}", flush=True)


def main():
    if os.environ.get("MALLOC_MMAP_MAX_") != "0":
        env = dict(os.environ, MALLOC_MMAP_MAX_="0", MALLOC_TRIM_THRESHOLD_=str(1 << 40))
        os.execve(sys.executable, [sys.executable] + sys.argv, env)
    names = sys.argv[1:] or list(PLAN)
    cache = {}
    for n in names:
        make(n, cache)


if __name__ == "__main__":
    main()

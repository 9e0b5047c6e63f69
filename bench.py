#!/usr/bin/env python3
"""TTT-E2E prefill benchmark on one MI355X.

One step = one full prefill (Algorithm 1 of the reading notes: every chunk's
forward, loss recording, backward into the fast MLPs and SGD update) over a
synthetic sequence of T tokens whose ids and weights are already in HBM.

Prints one JSON line: prefill tokens/s (whole job), ms per step, ms per 1K
tokens, the same for the eta = 0 / no-update sliding-window prefill, MFMA
utilisation of the whole step against the bf16 dense peak, a roofline entry
for the dominant kernel class (timed live with HIP events on the prefill's
stream) and the CPU oracle timed on a bounded sample on this host.
"""
import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kappa_sum(T, k):
    """sum_{p=0}^{T-1} min(p+1, k): attended keys over all queries (Eq. 1 of the notes)."""
    if T <= k:
        return T * (T + 1) // 2
    return k * (k + 1) // 2 + (T - k) * k


def chunk_pair_sum(T, b, k):
    """sum over chunk keys p of the chunk queries that attend p: min(s+n-p, k) per key."""
    tot = 0
    for s in range(0, T, b):
        n = min(b, T - s)
        tot += sum(min(n - i, k) for i in range(n))
    return tot


def algorithmic_flops(cfg, T, update=True):
    """Per-class algorithmic FLOPs of one prefill (multiply-add = 2; no recomputation,
    padding or masked-tile work counted)."""
    L, d, F, V, nu, k, b = cfg.n_layers, cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_update, cfg.window, cfg.chunk
    ks = kappa_sum(T, k)
    f = {
        "gemm_qkv": 6 * d * d * T * L,
        "attn_fwd": 4 * d * ks * L,
        "gemm_o_residual": 2 * d * d * T * L,
        "gemm_gate_up_swiglu": T * ((L - nu) * 4 * d * F + nu * 8 * d * F),
        "gemm_down_residual": T * ((L - nu) * 2 * d * F + nu * 4 * d * F),
        "gemm_lmhead_ce": 2 * d * V * T,
    }
    if update and nu > 0:
        nb = nu - 1
        f.update({
            "gemm_dn": 2 * d * V * T,
            "gemm_dhmid": T * (nb * 4 * d * F + 2 * d * F),
            "gemm_dw_sgd": T * nu * 6 * d * F,
            "gemm_dm": T * nb * 8 * d * F,
            "gemm_do": T * nb * 2 * d * d,
            "gemm_da": T * nb * 6 * d * d,
            "attn_bwd_dq": nb * 4 * d * ks,
            "attn_bwd_dkdv": nb * 4 * d * chunk_pair_sum(T, b, k),
        })
    return f


def head_single_pass(cfg, w):
    """Whether the library runs the head's loss and gradient in one pass for these weights:
    its create-time test, 2 * 1.01 sqrt(d) max|g_final| max_v |W_v| + ln V <= 126, which
    bounds every row's logit spread around its label's logit (only used here to book the
    head's FLOPs)."""
    import torch
    wn = float(torch.linalg.vector_norm(w["lm_head"].float(), dim=1).max())
    gm = float(w["final_norm"].float().abs().max())
    b = 1.01 * wn * gm * np.sqrt(cfg.d_model)
    return bool(np.isfinite(b) and 2 * b + np.log(cfg.vocab) <= 126.0)


def recompute_flops(cfg, T, update=True, single_pass=True):
    """FLOPs the path spends again on purpose and that are not algorithmic: none when the
    head runs its loss and gradient in one pass; otherwise the head backward computes each
    vocabulary slab's logits a second time after the cross-entropy pass (2 d V per token)."""
    if not update or cfg.n_update == 0 or single_pass:
        return {}
    return {"gemm_lmhead_ce": 2 * cfg.d_model * cfg.vocab * T}


def algorithmic_bytes(cfg, T, update=True):
    """Per-class HBM bytes of one prefill for the bandwidth-bound kernels: what each kernel
    must read and write given the stored layouts (fp32 residual stream and projections,
    16-bit activations, fp32 master fast weights), counted once; no re-reads, padding or
    cache effects.  The forward residual products' split-K partials are counted where they
    are reduced (in the RMSNorm that follows each product, with the planner's split); the
    backward's split-K reductions and the attention merges are not listed.  `update_in_gemm_dw_sgd` is the SGD step fused into the
    weight-gradient GEMM's epilogue (read and write the fp32 master, write the 16-bit
    forward copy and the transposed copy the backward reads)."""
    L, d, F, V, nu, H = cfg.n_layers, cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_update, cfg.n_heads
    a = 2 if cfg.dtype == "bf16" else 4          # activation / working-copy element size
    hilo = 2 if cfg.dtype == "bf16" else 1       # 16-bit forward copy is hi + lo
    nb = max(nu - 1, 0)                          # blocks whose attention is back-propagated
    P = 2 * ((V + 127) // 128)                   # CE partials per row
    n_chunks = (T + cfg.chunk - 1) // cfg.chunk
    # rmsnorm: read fp32 row, write the normalised row; the saved inputs of back-propagated norms;
    # the norms after the O and down products also apply those products' split-K partials
    # (read each fp32 partial, write the updated residual row)
    def split_k(M, N, K):  # the GEMM planner's split for a residual product (16-bit operands)
        def rnd(sp):
            if sp < 2:
                return 1
            per = -(-(-(-K // sp)) // 64) * 64
            return -(-K // per)
        t256 = -(-M // 256) * -(-N // 256)
        if t256 >= 200:
            return 1
        s256 = min(-(-240 // t256), K // 1024, 8)
        if s256 >= 4:
            return rnd(s256)
        tiles = -(-M // 128) * -(-N // 128)
        if tiles >= 256:
            return 1
        return rnd(min(-(-400 // tiles), K // 512, 4))
    b_rows = cfg.chunk
    # the frozen blocks below the updated ones run ahead over groups of 8192 to 16384 tokens
    # (the library picks the count per shape; only whether there is more than one chunk's
    # worth matters here) with unsplit products; their outputs are then copied into each
    # chunk's residual rows (fp32 read + write, timed with the embedding)
    G = min(max(1, 8192 // cfg.chunk) * cfg.chunk, n_chunks * cfg.chunk)
    grouped = (L - nu) > 0 and G > cfg.chunk
    sp_o = split_k(b_rows, d, d)
    sp_dn = split_k(b_rows, d, F)
    sp_df = split_k(b_rows, d, (3 if a == 2 else 2) * F)
    n_o = nu if grouped else L                   # layers whose O product is split by rows of a chunk
    red = n_o * (sp_o * 4 + 4) * d if sp_o > 1 else 0
    red += (L - nu) * (sp_dn * 4 + 4) * d if sp_dn > 1 and not grouped else 0
    red += nu * (sp_df * 4 + 4) * d if sp_df > 1 else 0
    rms = (2 * L + 1) * (4 + a) * d + ((nb + nu + 1) * 4 * d if update and nu > 0 else 0) + red
    # QK-norm + RoPE: read fp32 q, k, v; write q and the ring's K and V^T; the backward's
    # copies (V, K^T, 16-bit K) of back-propagated blocks, and with the update q copies
    rope = L * (12 + 3 * a) * d + nb * 3 * a * d + (nb * 2 * a * d if update else 0)
    # the head's row kernels (timed as one class with the loss reduce): the per-row shift reads
    # the normalised row and the label's head row (the 16-bit forward copy: 2 bytes in bf16
    # workloads) and writes 4 bytes; with updates the finish reads and writes the fp32 dn row
    # and reads the label's head row again
    wh = 2 if cfg.dtype == "bf16" else 4
    head_rows = (a + wh) * d + 8 + ((8 + wh) * d + 12 if update and nu > 0 else 0)
    b = {"embed": T * (a + 4) * d + (T * 8 * d if grouped else 0), "rmsnorm": T * rms, "qknorm_rope_ring": T * rope,
         "ce_reduce": T * (8 * P + 12 + head_rows)}
    if update and nu > 0:
        b.update({
            # final norm (dy, x, out fp32 + 16-bit) and two norms per back-propagated block (+ dh_in)
            "rmsnorm_bwd": T * ((12 + a) * d + 2 * nb * (16 + a) * d),
            # gate/up pre-activations and dhmid in, dgate/dup out (2F units above the lowest block)
            "swiglu_bwd": T * 5 * a * (nb * 2 * F + F),
            "qknorm_rope_bwd": T * nb * (24 + 3 * a) * d,
            "attn_bwd_pre": T * nb * (3 * a * d + 4 * H),
            # activations dy, hmid, dgu, m (read + write) per token
            "transpose": nu * T * 2 * a * (2 * d + 3 * F),
            # fp32 master read + write, the forward copy (hi | lo) and the backward's
            # transposed copy, written by the weight-gradient GEMM's epilogue
            "update_in_gemm_dw_sgd": n_chunks * nu * 3 * d * F * (8 + hilo * a + a),
        })
    return b


def steady_start(cfg):
    """First position of the first chunk whose window is full (chunk index ceil(k/b)),
    or None when the sequence has no such chunk."""
    s = -(-cfg.window // cfg.chunk) * cfg.chunk
    return s if s < cfg.seq_len else None


def gpu_bench(cfg, steps, warmup, profile=True, gains=None):
    """Times the prefill of cfg's sequence with inner updates and with eta = 0 (no
    backward, no update), and, when the sequence has chunks with a full window, the
    prefill of its first s tokens (s = ceil(k/b) b): the difference prices the
    steady-state chunks (chunk index >= k/b) alone."""
    import torch
    from ttt_inputs import make_weights_torch, make_tokens
    from test_lm_prefill_amd import Session
    from test_lm_prefill_amd.ttt import TTT_NO_UPDATE

    T = cfg.seq_len
    log(f"[bench] workload {cfg.name}: L={cfg.n_layers} d={cfg.d_model} T={T} b={cfg.chunk} k={cfg.window}")
    t0 = time.time()
    w = make_weights_torch(cfg, "cuda", seed=0, gains=gains)
    tok_np = make_tokens(cfg, seed=1)
    tok = torch.from_numpy(tok_np).cuda()
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    sess = Session(cfg, w, max_tokens=T)
    stream = torch.cuda.current_stream()

    def timed(flags, K, W, t=tok):
        for i in range(W):
            sess.prefill(t, flags=flags, want_fast=False, check=False)
            torch.cuda.synchronize()
            log(f"[bench] warmup {i + 1}/{W} flags={flags} T={t.numel() - 1} done")
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            sess.prefill(t, flags=flags, want_fast=False, check=False)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        log(f"[bench] timed {K} steps flags={flags} T={t.numel() - 1}: {ms / K:.2f} ms/step")
        return ms / K

    res = {"ms_ttt": timed(0, steps, warmup), "head_single_pass": head_single_pass(cfg, w)}
    losses, _ = sess.prefill(tok, want_fast=False, check=True)
    res["mean_loss"] = float(losses.mean().item())
    res["ms_swa"] = timed(TTT_NO_UPDATE, steps, 1)
    s0 = steady_start(cfg)
    if s0 is not None:
        head = tok[:s0 + 1].contiguous()
        res["steady_s0"] = s0
        res["ms_ttt_head"] = timed(0, max(2, steps), 1, head)
        res["ms_swa_head"] = timed(TTT_NO_UPDATE, max(2, steps), 1, head)
    res["kt"] = {}
    if profile:
        sess.set_kernel_timing(True)
        sess.prefill(tok, want_fast=False, check=False)
        torch.cuda.synchronize()
        res["kt"] = sess.kernel_times()
        sess.set_kernel_timing(False)
        log("[bench] kernel timing pass done")
    sess.close()
    del w
    torch.cuda.empty_cache()
    res["tok_np"] = tok_np
    return res


def time_prefill(cfg, flags, steps, warmup, n_seq=1):
    """ms per prefill of cfg's own sequence with the given flags (fresh session); with
    n_seq > 1, of a batch of n_seq sequences (the workload's stream and n_seq-1 more seeds)."""
    import torch
    from ttt_inputs import make_weights_torch, make_tokens
    from test_lm_prefill_amd import Session
    w = make_weights_torch(cfg, "cuda", seed=0)
    if n_seq == 1:
        tok = torch.from_numpy(make_tokens(cfg, seed=1)).cuda()
    else:
        tok = torch.from_numpy(np.stack([make_tokens(cfg, seed=1 + i) for i in range(n_seq)])).cuda()
    sess = Session(cfg, w, max_tokens=cfg.seq_len, n_seq=n_seq)
    stream = torch.cuda.current_stream()
    try:
        for _ in range(warmup):
            sess.prefill(tok, flags=flags, want_fast=False, check=False)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            sess.prefill(tok, flags=flags, want_fast=False, check=False)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
    finally:
        sess.close()
        del w, tok
        torch.cuda.empty_cache()
    log(f"[bench] {cfg.name} B={n_seq} T={cfg.seq_len} k={cfg.window} n_u={cfg.n_update} flags={flags}: {ms:.1f} ms")
    return ms


def suite_full_attention(steps, warmup):
    """Full-attention prefill baseline at the 2.7B shape: the window covers the whole
    sequence (k >= T, a linear KV cache of T + b rows), no fast MLPs and no inner
    updates, i.e. a plain causal Transformer of the same size; timed beside the
    TTT-E2E prefill (k = 8K, inner updates) of the same T.  The notes quote a 2.7x
    speed-up of TTT-E2E over full attention at 128K on one H100 (section 11.1)."""
    from ttt_inputs import get
    from test_lm_prefill_amd.ttt import TTT_NO_UPDATE
    rows = []
    for name in ("2.7b_8k", "2.7b_32k", "2.7b_128k"):
        cfg = get(name)
        T = cfg.seq_len
        ms_ttt = time_prefill(cfg, 0, steps, warmup)
        fa = cfg.with_(name=name + "_full_attention", window=-(-T // 64) * 64, n_update=0)
        ms_fa = time_prefill(fa, TTT_NO_UPDATE, steps, warmup)
        rows.append({"seq_len": T, "ttt_e2e_ms": round(ms_ttt, 1), "full_attention_ms": round(ms_fa, 1),
                     "ttt_e2e_ms_per_1k": round(ms_ttt * 1024 / T, 3),
                     "full_attention_ms_per_1k": round(ms_fa * 1024 / T, 3),
                     "speedup_ttt_over_full": round(ms_fa / ms_ttt, 3)})
    return {"suite": "full_attention_baseline", "shape": "2.7b", "rows": rows}


def suite_sweep(steps, warmup):
    """ms per 1K tokens of the TTT-E2E prefill at the 760M shape (T = 128K, b = 1K) over
    the number of updated blocks n_u (k = 8K) and the window k (n_u = 6)."""
    from ttt_inputs import get
    base = get("760m")
    rows = []
    for nu, k in [(1, 8192), (3, 8192), (6, 8192), (12, 8192), (6, 2048), (6, 4096), (6, 16384)]:
        cfg = base.with_(name=f"760m_nu{nu}_k{k}", n_update=nu, window=k)
        ms = time_prefill(cfg, 0, steps, warmup)
        rows.append({"n_update": nu, "window": k, "ms": round(ms, 1),
                     "ms_per_1k": round(ms * 1024 / cfg.seq_len, 3)})
    return {"suite": "n_update_and_window_sweep", "shape": "760m", "seq_len": base.seq_len, "rows": rows}


def suite_batch(steps, warmup):
    """Batched independent sequences at the 2.7B shape with 131072 tokens per call
    (B = 131072 / T sequences of T tokens, each with its own fast weights and window),
    against the same T one sequence per call."""
    from ttt_inputs import get
    rows = []
    for name, B in (("2.7b_8k", 16), ("2.7b_32k", 4)):
        cfg = get(name)
        T = cfg.seq_len
        ms1 = time_prefill(cfg, 0, steps, warmup)
        msb = time_prefill(cfg, 0, steps, warmup, n_seq=B)
        rows.append({"seq_len": T, "n_seq": B, "one_seq_ms": round(ms1, 1),
                     "one_seq_tokens_per_s": round(T / (ms1 / 1e3), 1), "batch_ms": round(msb, 1),
                     "batch_tokens_per_s": round(B * T / (msb / 1e3), 1),
                     "speedup": round(B * ms1 / msb, 3)})
    return {"suite": "batched_sequences", "shape": "2.7b", "tokens_per_batch": 131072, "rows": rows}


def suite_decode(steps, warmup, n_decode=2048, prompt_cfg="2.7b_8k"):
    """Algorithm 3 at the 2.7B shape: prefill an 8K prompt, then greedy-decode n_decode
    ids one call per position, each bracketed by HIP events on the decode stream.
    Steps whose call closes a decode chunk also run that chunk's update (the chunk
    forward again, its backward and the SGD step): the stall at update boundaries."""
    import torch
    from ttt_inputs import get, make_weights_torch, make_tokens
    from test_lm_prefill_amd import Session
    cfg = get(prompt_cfg)
    T = cfg.seq_len
    w = make_weights_torch(cfg, "cuda", seed=0)
    tok = torch.from_numpy(make_tokens(cfg, seed=1)).cuda()
    sess = Session(cfg, w, max_tokens=T + n_decode)
    stream = torch.cuda.current_stream()
    try:
        sess.prefill(tok, want_fast=False, check=False)
        sess.decode(cfg.chunk + 8, want_fast=False, check=False)    # warm-up: captures both graphs
        sess.prefill(tok, want_fast=False, check=False)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_decode)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for j in range(n_decode):
            ev[j][0].record(stream)
            sess.decode(1, want_fast=False, check=False)
            ev[j][1].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        total = t0.elapsed_time(t1)
    finally:
        sess.close()
        del w, tok
        torch.cuda.empty_cache()
    upd = np.arange(n_decode)[(np.arange(n_decode) + 1) % cfg.chunk == 0]
    plain = np.setdiff1d(np.arange(n_decode), upd)
    return {"suite": "decode_periodic_updates", "shape": "2.7b", "prompt": T, "decoded": n_decode,
            "chunk": cfg.chunk, "mode": "greedy",
            "ms_per_token_median": round(float(np.median(ms[plain])), 3),
            "ms_per_token_p90": round(float(np.percentile(ms[plain], 90)), 3),
            "update_step_ms_median": round(float(np.median(ms[upd])), 2) if len(upd) else None,
            "stall_ms": round(float(np.median(ms[upd]) - np.median(ms[plain])), 2) if len(upd) else None,
            "tokens_per_s_including_updates": round(n_decode / (total / 1e3), 1),
            "total_ms": round(total, 1)}


def profile_pass(cfg):
    """For hardware-counter runs: one kernel of known traffic, then one prefill.

    The calibration is torch's elementwise negation of 2**28 fp32 values, which
    reads 1 GiB and writes 1 GiB once each; a counter's reading for it gives the
    scale from counter units to bytes.  The prefill launches its kernels one by
    one (no graph replay; the kernels are the same), because the profiler's
    counter collection does not follow graph launches.
    """
    import torch
    from ttt_inputs import make_weights_torch, make_tokens
    from test_lm_prefill_amd import Session
    w = make_weights_torch(cfg, "cuda", seed=0)
    tok = torch.from_numpy(make_tokens(cfg, seed=1)).cuda()
    sess = Session(cfg, w, max_tokens=cfg.seq_len)
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    log("[bench] calibration kernel done")
    from test_lm_prefill_amd.ttt import TTT_NO_GRAPH
    sess.prefill(tok, flags=TTT_NO_GRAPH, want_fast=False, check=False)
    torch.cuda.synchronize()
    log("[bench] profile prefill done")
    sess.close()
    print(json.dumps({"profile_pass": cfg.name, "calibration_bytes_read": n * 4, "calibration_bytes_written": n * 4}),
          flush=True)


def source_digest(paths):
    import hashlib
    hsh = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the counter runs kept under profiles/, or None when
    none is stored for this kernel and workload or its sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- (\w+): (\S+)", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    srcs = fields.get("sources", "").split(",")
    if not srcs or fields.get("digest") != source_digest(srcs):
        return None
    return float(fields["bytes_per_launch"])


def host_info():
    """CPU model, logical / physical / usable cores and the BLAS numpy calls."""
    info = {"cpu_model": None, "logical_cores": os.cpu_count(), "physical_cores": None,
            "usable_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}
    try:
        phys, pid, cid = set(), None, None
        with open("/proc/cpuinfo") as f:
            for line in f:
                key = line.split(":", 1)[0].strip()
                if key == "model name" and info["cpu_model"] is None:
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                elif key == "physical id":
                    pid = line.split(":", 1)[1].strip()
                elif key == "core id":
                    cid = line.split(":", 1)[1].strip()
                elif not line.strip():
                    if cid is not None:
                        phys.add((pid, cid))
                    pid, cid = None, None
        if cid is not None:
            phys.add((pid, cid))
        info["physical_cores"] = len(phys) or None
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = {"vendor": blas[0].get("internal_api"), "version": blas[0].get("version"),
                            "threads": blas[0].get("num_threads"),
                            "architecture": blas[0].get("architecture")}
    except Exception:
        pass
    return info


def cpu_baseline(cfg, tok_np, gains=None, seed=7, n_max=128):
    """The oracle (numpy float64, as it is) on a bounded sample of the same workload.

    Workloads with chunks whose window is full: the first n_max positions of one such
    steady-state chunk (chunk index ceil(k/b)), run as a chunk of their own (forward,
    losses, backward and the SGD step; the work per position is that of the full chunk:
    every query sees k keys, every product has the same shapes per row), with the k-1
    cached positions per layer filled with seeded random keys and values in place of
    the earlier chunks' own (their values do not change the work).  Workloads without
    such a chunk: the whole prefill when it is short (up to 4 chunks), else the first
    n_max positions of its last chunk the same way.
    """
    from ttt_inputs import make_weights_torch
    from oracle.ttt_oracle import Oracle, sgd_step
    import torch
    t0 = time.time()
    w = make_weights_torch(cfg, "cuda" if torch.cuda.is_available() else "cpu", seed=0, gains=gains)
    wn = {k: v.float().cpu().numpy() for k, v in w.items()}
    del w
    torch.cuda.empty_cache()
    log(f"[bench] cpu baseline: weights on host in {time.time() - t0:.1f}s")
    orc = Oracle(cfg, wn)
    T, b, k = cfg.seq_len, cfg.chunk, cfg.window
    hi = host_info()
    threads = (hi.get("blas") or {}).get("threads") or hi["usable_cores"]
    s0 = steady_start(cfg)
    if s0 is None and cfg.n_chunks <= 4:
        t1 = time.time()
        orc.prefill(tok_np[:T + 1])
        dt = time.time() - t1
        n, what = T, f"the whole prefill ({cfg.n_chunks} chunks of {b})"
    else:
        if s0 is None:
            s0 = (cfg.n_chunks - 1) * b
            kind = "the last chunk"
        else:
            kind = "one steady-state chunk (chunk index ceil(k/b))"
        n = min(b, T - s0, n_max)
        rng = np.random.default_rng(seed)
        lo = max(0, s0 - k + 1)
        shape = (s0 - lo, cfg.n_heads, cfg.head_dim)
        cache = [{"pos": np.arange(lo, s0, dtype=np.int64), "k": rng.standard_normal(shape),
                  "v": 0.05 * rng.standard_normal(shape)} for _ in range(cfg.n_layers)]
        W = orc.init_fast()
        t1 = time.time()
        _, saved, _ = orc.chunk_forward(W, cache, tok_np[s0:s0 + n], tok_np[s0 + 1:s0 + n + 1], s0)
        if cfg.n_update > 0:
            G = orc.chunk_grad(W, saved)
            W = [[sgd_step(x, g, cfg.eta) for x, g in zip(ws, gs)] for ws, gs in zip(W, G)]
        dt = time.time() - t1
        what = (f"the first {n} positions of {kind}, run as a chunk of their own: positions {s0}..{s0 + n - 1} "
                f"with {s0 - lo} cached positions per layer (seeded random keys and values), forward, losses, "
                f"backward and one SGD step")
    log(f"[bench] cpu baseline: {n} tokens in {dt:.1f}s")
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "ms_per_1k_tokens": round(dt * 1e3 * 1024 / n, 1),
            "projected_whole_prefill_s": round(dt * T / n, 1),  # every chunk priced as a steady-state one
            "sample": f"{what}; numpy float64; {dt:.1f} s",
            "host": hi}


def attention_path(cfg, gains):
    """Which forward attention kernel the library picks for these QK-norm gains (its
    rule: bound B = 1.01 max|g_q| max|g_k| sqrt(hd) log2(e) of the scaled scores in
    log2 units; fp16 bounded softmax for B <= 14.5, bf16 bounded for B <= 48, else the
    online-max kernel), per layer, counted."""
    if cfg.dtype != "bf16":
        return {"fp32 online max": cfg.n_layers}
    out = {}
    for l in range(cfg.n_layers):
        gq = 1.0 if gains is None else float(np.abs(gains[f"l{l}.q_norm"]).max())
        gk = 1.0 if gains is None else float(np.abs(gains[f"l{l}.k_norm"]).max())
        B = 1.01 * gq * gk * np.sqrt(cfg.head_dim) * 1.4426950408889634
        path = "fp16 bounded softmax" if B <= 14.5 else ("bf16 bounded softmax" if B <= 48 else "bf16 online max")
        out[path] = out.get(path, 0) + 1
    return out


def qk_gains(cfg, product):
    """Unit block-norm gains and QK-norm gains sqrt(product) each (bf16-rounded)."""
    from ttt_inputs.weights import tensor_specs, round_bf16_np
    g = {}
    for name, _, shape, kind in tensor_specs(cfg):
        if kind == "gain":
            v = np.sqrt(product) if name.endswith(("q_norm", "k_norm")) else 1.0
            g[name] = round_bf16_np(np.full(shape, v, dtype=np.float32))
    return g


def overhead_flops(cfg, T):
    """MFMA work the path does beyond the algorithmic count: the bf16 workloads' fast
    MLP forward runs over the hi | lo working copy, doubling the reduction of the fast
    gate/up (4 d F per token per fast block) and fast down (2 d F) products."""
    if cfg.dtype != "bf16" or cfg.n_update == 0:
        return {}
    return {"gemm_gate_up_swiglu": T * cfg.n_update * 4 * cfg.d_model * cfg.d_ff,
            "gemm_down_residual": T * cfg.n_update * 2 * cfg.d_model * cfg.d_ff}


def summarize(cfg, r, steps):
    """The per-workload figures from one gpu_bench result."""
    T = cfg.seq_len
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    flops = algorithmic_flops(cfg, T, update=True)
    total_tf = sum(flops.values()) / 1e12
    swa_tf = sum(algorithmic_flops(cfg, T, update=False).values()) / 1e12
    ov = overhead_flops(cfg, T)
    rflops = recompute_flops(cfg, T, update=True, single_pass=r.get("head_single_pass", True))
    out = {
        "ms_per_step": round(r["ms_ttt"], 3),
        "ms_per_1k_tokens": round(r["ms_ttt"] * 1024 / T, 4),
        "tokens_per_s": round(T / (r["ms_ttt"] / 1e3), 1),
        "mfma_util_pct": round(100 * total_tf / (r["ms_ttt"] / 1e3) / peak, 2),
        "algorithmic_tflop_per_step": round(total_tf, 2),
        "overhead_tflop_per_step": {"hilo_fast_forward": round(sum(ov.values()) / 1e12, 2),
                                    "head_backward_logits_recompute": round(sum(rflops.values()) / 1e12, 2)},
        "head_single_pass": r.get("head_single_pass"),
        "swa_only": {"ms_per_step": round(r["ms_swa"], 3), "ms_per_1k_tokens": round(r["ms_swa"] * 1024 / T, 4),
                     "tokens_per_s": round(T / (r["ms_swa"] / 1e3), 1),
                     "mfma_util_pct": round(100 * swa_tf / (r["ms_swa"] / 1e3) / peak, 2)},
        "ttt_over_swa": round(r["ms_ttt"] / r["ms_swa"], 3),
    }
    if "steady_s0" in r:
        n = T - r["steady_s0"]
        out["steady_state"] = {
            "chunks": f"{r['steady_s0'] // cfg.chunk}..{cfg.n_chunks - 1}",
            "ms_per_1k_tokens": round((r["ms_ttt"] - r["ms_ttt_head"]) * 1024 / n, 4),
            "swa_only_ms_per_1k_tokens": round((r["ms_swa"] - r["ms_swa_head"]) * 1024 / n, 4),
            "how": f"(prefill of T tokens - prefill of the first {r['steady_s0']}) / {n} tokens"}
    kt = r["kt"]
    kernels = {}
    if kt:
        hbm = algorithmic_bytes(cfg, T, update=True)
        tot_prof = sum(v[0] for v in kt.values())
        for nm, (ms, cnt) in sorted(kt.items(), key=lambda x: -x[1][0]):
            if cnt == 0:
                continue
            ent = {"ms": round(ms, 3), "launches": cnt, "share": round(ms / tot_prof, 4)}
            if nm in flops and ms > 0:
                ent["tflops"] = round(flops[nm] / 1e12 / (ms / 1e3), 1)
                ent["mfma_frac"] = round(flops[nm] / 1e12 / (ms / 1e3) / peak, 4)
            if nm in ov and ms > 0:  # the hi | lo work: its own entry, outside the algorithmic rate
                ent["overhead_tflop"] = round(ov[nm] / 1e12, 2)
                ent["tflops_incl_overhead"] = round((flops[nm] + ov[nm]) / 1e12 / (ms / 1e3), 1)
            if nm in rflops and ms > 0:
                ent["recompute_tflops"] = round(rflops[nm] / 1e12 / (ms / 1e3), 1)
            ub = hbm.get("update_in_gemm_dw_sgd") if nm == "gemm_dw_sgd" else None
            if (nm in hbm or ub) and ms > 0:
                by = ub if ub else hbm[nm]
                key = "update_" if ub else ""
                ent[key + "gbytes"] = round(by / 1e9, 3)
                ent[key + "gbps"] = round(by / 1e9 / (ms / 1e3), 1)
                ent[key + "hbm_frac"] = round(by / 1e9 / (ms / 1e3) / PEAK_HBM_GBS, 4)
            kernels[nm] = ent

        def util(names):
            f = sum(flops[nm] for nm in names if nm in kt)
            t = sum(kt[nm][0] for nm in names if nm in kt)
            return round(f / 1e12 / (t / 1e3) / peak, 4) if t > 0 else None
        out["mfma_frac_by_family"] = {
            "gemm": util([nm for nm in flops if nm.startswith("gemm_")]),
            "attention": util([nm for nm in flops if nm.startswith("attn_")])}
        out["hbm_gbps"] = {nm: kernels[nm].get("gbps") or kernels[nm].get("update_gbps")
                           for nm in ("rmsnorm", "rmsnorm_bwd", "ce_reduce", "gemm_dw_sgd") if nm in kernels}
    out["kernels"] = kernels
    return out, flops, peak


def roofline_entry(cfg, r, flops, peak):
    kt = r["kt"]
    if not kt:
        return None
    dom = max((nm for nm in kt if nm in flops and kt[nm][1] > 0), key=lambda nm: kt[nm][0])
    ms_d, n_d = kt[dom]
    per_launch = flops[dom] / n_d
    achieved = per_launch / 1e12 / (ms_d / n_d / 1e3)
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": stored_traffic(dom, cfg.name), "kernel": dom,
            "flop_per_launch": per_launch, "avg_launch_ms": round(ms_d / n_d, 4)}


def precision(cfg, gains):
    if cfg.dtype != "bf16":
        return "fp32", {"all": "fp32"}
    return "fp16", {"weights": "bf16 values", "forward_gemm_operands": "fp16",
                    "attention_forward": attention_path(cfg, gains),
                    "mlp_backward_operands": "fp16 (loss scaled by 2^12)",
                    "attention_and_vocab_backward_operands": "bf16", "accumulate": "fp32",
                    "fast_weight_master": "fp32", "residual_stream_and_losses": "fp32"}


# every listed workload but the headline 2.7B, T = 131072 one
OTHER_WORKLOADS = ("tiny", "125m", "760m", "1.3b_b256", "1.3b_b1024", "1.3b_b4096", "2.7b_8k", "2.7b_32k")


def suite_configs(steps, warmup, with_cpu=True):
    """Every listed workload besides the headline one: whole-sequence and steady-state
    ms per 1K tokens with inner updates and with eta = 0, MFMA fractions of the GEMM and
    attention families, HBM rates of the norm, CE and update kernels, and the oracle on
    its bounded sample."""
    from ttt_inputs import get
    rows = []
    for name in OTHER_WORKLOADS:
        cfg = get(name)
        r = gpu_bench(cfg, steps, warmup, profile=True)
        row, _, _ = summarize(cfg, r, steps)
        row = {"workload": name, "seq_len": cfg.seq_len, "chunk": cfg.chunk, "window": cfg.window,
               "n_update": cfg.n_update, **row}
        row.pop("kernels")
        row["dtype"] = precision(cfg, None)[0]
        row["mean_loss"] = round(r["mean_loss"], 4)
        if with_cpu:
            row["cpu_baseline"] = cpu_baseline(cfg, r["tok_np"])
        rows.append(row)
        log(f"[bench] {name}: {row['ms_per_1k_tokens']} ms/1K (swa {row['swa_only']['ms_per_1k_tokens']})")
    return {"suite": "workloads", "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="2.7b_128k")
    ap.add_argument("--qk-gain", type=float, default=None,
                    help="QK-norm gains sqrt(G) for q and k (product G) instead of unit gains")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="run a calibration kernel and one prefill only (for counter runs)")
    ap.add_argument("--suite", choices=["full_attention", "sweep", "decode", "batch", "workloads"],
                    help="instead of the benchmark line: the full-attention baseline at the 2.7B shape, "
                         "the n_update / window sweep at the 760M shape, decoding with periodic "
                         "updates after an 8K prompt at the 2.7B shape, batched sequences at 131072 "
                         "tokens per call at the 2.7B shape, or every other listed workload (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: a TTT prefill sequence is a recurrence over chunks and "
              "independent sequences shard with no communication; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    from ttt_inputs import get
    cfg = get(args.config)
    if args.profile_pass:
        profile_pass(cfg)
        return
    if args.suite:
        if args.suite == "workloads":
            print(json.dumps(suite_configs(args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)), flush=True)
            return
        fn = {"full_attention": suite_full_attention, "sweep": suite_sweep, "decode": suite_decode,
              "batch": suite_batch}[args.suite]
        print(json.dumps(fn(args.steps, args.warmup)), flush=True)
        return
    T = cfg.seq_len
    gains = qk_gains(cfg, args.qk_gain) if args.qk_gain is not None else None
    r = gpu_bench(cfg, args.steps, args.warmup, profile=not args.no_kernel_timing, gains=gains)
    summ, flops, peak = summarize(cfg, r, args.steps)
    roof = roofline_entry(cfg, r, flops, peak)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, r["tok_np"], gains=gains)
    dtype, prec = precision(cfg, gains)
    out = {
        "metric": "TTT prefill tokens/s and ms per 1K tokens at 128K ctx; MFMA util %",
        "value": round(T / (r["ms_ttt"] / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": summ.pop("ms_per_step"),
        "ms_per_1k_tokens": summ.pop("ms_per_1k_tokens"),
        "mfma_util_pct": summ.pop("mfma_util_pct"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded Zipf+span-copy ids, seeded random-init weights)",
        "precision": prec,
        "config": {"workload": cfg.name + (f"_qkgain{args.qk_gain:g}" if gains is not None else ""),
                   "n_layers": cfg.n_layers, "d_model": cfg.d_model, "n_heads": cfg.n_heads,
                   "d_ff": cfg.d_ff, "vocab": cfg.vocab, "seq_len": T, "window": cfg.window, "chunk": cfg.chunk,
                   "n_update": cfg.n_update, "eta": cfg.eta,
                   "qk_gain_product": args.qk_gain if gains is not None else 1.0},
        "mean_loss": round(r["mean_loss"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    summ.pop("tokens_per_s")
    out.update(summ)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

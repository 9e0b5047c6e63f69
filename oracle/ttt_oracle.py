"""CPU oracle for the TTT-E2E prefill: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never calls it and shares no code with it.

What it computes (zhongzhuzhou.org notes "TTT-E2E 阅读笔记", section 7,
Algorithm 1, with Eq. (9) of section 5 and Eq. (3) of section 3):

  * copy the fast weights W <- W_init for the sequence (Alg. 1 step 1);
  * read the context in chunks of b positions in time order (step 3);
  * predict every target of the chunk with the current W and the frozen
    parameters phi, under a causal sliding-window mask (steps 3.1, 3.2);
  * record the per-token losses BEFORE any use of their labels (step 3.3);
  * take the gradient of the chunk's mean loss A_i(W) (Eq. 9) with respect to
    the fast weights only (step 3.4) and one SGD step W <- W - eta * grad
    (step 3.5, Eq. 9);
  * keep only the attention state the window still needs (step 3.6);
  * after a prefill, generation with periodic updates (Algorithm 3): feed one
    position at a time, take the next id from the prediction (or as given), and
    once a chunk of b positions has all its targets, update W on that chunk as
    Algorithm 1 does (``Oracle.decode``).

Model (pre-norm Transformer with sliding-window attention and QK-norm; the
jdon.com page, "架构极简" paragraph and the basic-recipe paragraph; the notes,
section 6, for the fast MLP of the last quarter of blocks and its static
companion branch).  The pages leave the block internals open; the readings used
are: RMSNorm everywhere, per-head RMSNorm of q and k with learned gains applied
before a half-split rotary embedding, SwiGLU MLPs, untied output head, the fast
and static SwiGLU of an updated block summed on one shared pre-MLP norm, cached
keys/values computed with the weights of their own chunk and held constant in
the gradient, plain SGD with a fixed step, N updates for N chunks (the last one
changes no recorded loss), and a short last chunk averaged over its own size.

Everything runs in numpy float64 by default (``dtype=np.float32`` is a switch).
The backward pass is written out by hand.  Matrix products use numpy's BLAS.
"""
import numpy as np


# --------------------------------------------------------------------------- pieces
def rmsnorm(x, g, eps):
    """y = x * (mean(x^2) + eps)^-1/2 * g over the last axis; returns (y, r)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g, r


def rmsnorm_bwd(dy, x, r, g):
    """Gradient of rmsnorm w.r.t. x, given dy, the input x and the saved r."""
    gdy = dy * g
    return r * gdy - x * (r ** 3) * np.mean(x * gdy, axis=-1, keepdims=True)


def rope_tables(pos, hd, theta, dtype):
    """cos/sin of angle_i = p * theta^(-2i/hd), i < hd/2, computed in float64."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, cos, sin):
    """Half-split rotation of pairs (i, i + hd/2); x is [n, H, hd]."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation (rotation by the negative angle)."""
    h = dy.shape[-1] // 2
    d1, d2 = dy[..., :h], dy[..., h:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def dsilu(z):
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu(m, wg, wu, wd):
    """(silu(m Wg^T) * (m Wu^T)) Wd^T; returns output and (G, U, Hmid)."""
    G = m @ wg.T
    U = m @ wu.T
    Hm = silu(G) * U
    return Hm @ wd.T, (G, U, Hm)


def logsumexp(z):
    mx = np.max(z, axis=-1, keepdims=True)
    return (mx + np.log(np.sum(np.exp(z - mx), axis=-1, keepdims=True)))[..., 0]


def sgd_step(w, g, eta):
    """Inner update of Eq. (9): W_i = W_{i-1} - eta * grad."""
    return w - eta * g


# --------------------------------------------------------------------------- model
class Oracle:
    """Holds phi (frozen) and runs Algorithm 1 on a token sequence.

    ``weights`` maps names to arrays (any float dtype; values are cast to the
    working dtype where used).  ``cfg`` needs n_layers, d_model, n_heads,
    head_dim, d_ff, vocab, window, chunk, n_update, eta, rms_eps, rope_theta.
    """

    def __init__(self, cfg, weights, dtype=np.float64):
        self.cfg = cfg
        self.w = weights
        self.dt = dtype
        self.L = cfg.n_layers
        self.nu = cfg.n_update
        self.first_fast = self.L - self.nu
        self.key_count = 0          # instrumentation: total (query, key) pairs scored

    def p(self, name):
        return self.w[name].astype(self.dt, copy=False)

    def init_fast(self):
        """W <- W_init: a private copy for this sequence (Alg. 1 step 1)."""
        return [[self.p(f"fast{u}.w_gate").copy(), self.p(f"fast{u}.w_up").copy(),
                 self.p(f"fast{u}.w_down").copy()] for u in range(self.nu)]

    def empty_cache(self):
        """Bounded attention state per layer: positions, rotated keys, values."""
        c = self.cfg
        z = np.zeros((0, c.n_heads, c.head_dim), dtype=self.dt)
        return [{"pos": np.zeros(0, dtype=np.int64), "k": z, "v": z} for _ in range(self.L)]

    # ---------------------------------------------------------------- attention
    def window_mask(self, pos_q, pos_k):
        """Causal sliding window: query p sees keys j with p-k < j <= p."""
        return (pos_k[None, :] <= pos_q[:, None]) & (pos_k[None, :] > pos_q[:, None] - self.cfg.window)

    def head_probs(self, q_h, K_h, valid):
        """Softmax over the visible keys of one head: P = softmax(q k^T / sqrt(hd))."""
        s = (q_h @ K_h.T) * (1.0 / np.sqrt(self.cfg.head_dim))
        s = np.where(valid, s, -np.inf)
        s = s - np.max(s, axis=-1, keepdims=True)
        e = np.exp(s)
        return e / np.sum(e, axis=-1, keepdims=True)

    def attention(self, qh, pos_q, K, V, pos_k):
        """Causal sliding-window attention of the chunk's queries over K, V."""
        c = self.cfg
        valid = self.window_mask(pos_q, pos_k)
        self.key_count += int(valid.sum())
        o = np.empty_like(qh)
        for h in range(c.n_heads):
            o[:, h, :] = self.head_probs(qh[:, h, :], K[:, h, :], valid) @ V[:, h, :]
        return o

    def attention_bwd(self, do, qh, K, V, pos_q, pos_k, n_old):
        """Gradients w.r.t. the queries and the chunk's own keys/values.

        The probabilities are recomputed head by head with the forward's own
        function (nothing of size heads x queries x keys is kept).  Keys and
        values of earlier chunks (the first n_old rows of K, V) are constants of
        the current step, so only the chunk rows get gradients.
        """
        c = self.cfg
        scale = 1.0 / np.sqrt(c.head_dim)
        valid = self.window_mask(pos_q, pos_k)
        dq = np.empty_like(qh)
        nk = K.shape[0] - n_old
        dk = np.empty((nk, c.n_heads, c.head_dim), dtype=self.dt)
        dv = np.empty_like(dk)
        for h in range(c.n_heads):
            Ph = self.head_probs(qh[:, h, :], K[:, h, :], valid)
            dP = do[:, h, :] @ V[:, h, :].T
            Drow = np.sum(Ph * dP, axis=-1, keepdims=True)
            dS = Ph * (dP - Drow)
            dq[:, h, :] = (dS @ K[:, h, :]) * scale
            dk[:, h, :] = (dS[:, n_old:].T @ qh[:, h, :]) * scale
            dv[:, h, :] = Ph[:, n_old:].T @ do[:, h, :]
        return dq, dk, dv

    # ---------------------------------------------------------------- one chunk
    def chunk_forward(self, W, cache, x_in, labels, pos0, consume=False):
        """Forward of one chunk with fast weights W and attention state `cache`.

        Returns (losses, saved, new_cache).  `cache` is not modified unless
        `consume` is set: then each layer's old entry is dropped once the layer
        is done (the caller hands the state over; only memory use changes).
        """
        c = self.cfg
        n = len(x_in)
        H, hd, eps = c.n_heads, c.head_dim, c.rms_eps
        pos = np.arange(pos0, pos0 + n, dtype=np.int64)
        cos, sin = rope_tables(pos, hd, c.rope_theta, self.dt)
        h = self.w["tok_emb"][x_in].astype(self.dt)
        saved = {"layers": {}, "pos": pos, "cos": cos, "sin": sin}
        new_cache = []
        for l in range(self.L):
            pre = f"l{l}."
            h_in = h
            a, r1 = rmsnorm(h, self.p(pre + "attn_norm"), eps)
            q = (a @ self.p(pre + "wq").T).reshape(n, H, hd)
            k = (a @ self.p(pre + "wk").T).reshape(n, H, hd)
            v = (a @ self.p(pre + "wv").T).reshape(n, H, hd)
            qn, rq = rmsnorm(q, self.p(pre + "q_norm"), eps)
            kn, rk = rmsnorm(k, self.p(pre + "k_norm"), eps)
            qh = rope(qn, cos, sin)
            kh = rope(kn, cos, sin)
            K = np.concatenate([cache[l]["k"], kh], axis=0)
            V = np.concatenate([cache[l]["v"], v], axis=0)
            pos_k = np.concatenate([cache[l]["pos"], pos])
            o = self.attention(qh, pos, K, V, pos_k)
            h1 = h + o.reshape(n, -1) @ self.p(pre + "wo").T
            m, r2 = rmsnorm(h1, self.p(pre + "mlp_norm"), eps)
            ys, acts_s = swiglu(m, self.p(pre + "w_gate"), self.p(pre + "w_up"), self.p(pre + "w_down"))
            y = ys
            acts_f = None
            if l >= self.first_fast:
                wg, wu, wd = W[l - self.first_fast]
                yf, acts_f = swiglu(m, wg, wu, wd)
                y = ys + yf
            h = h1 + y
            if l >= self.first_fast:
                saved["layers"][l] = dict(h_in=h_in, r1=r1, q=q, k=k, v=v, rq=rq, rk=rk, qh=qh,
                                          K=K, V=V, pos_k=pos_k, n_old=len(cache[l]["pos"]), o=o,
                                          h1=h1, r2=r2, m=m, acts_s=acts_s, acts_f=acts_f)
            # Alg. 1 step 3.6: keep only what the window still needs.
            nxt = pos0 + n
            keep_mask = pos_k > nxt - c.window
            new_cache.append({"pos": pos_k[keep_mask], "k": K[keep_mask], "v": V[keep_mask]})
            if consume:
                cache[l] = None
        nf, rf = rmsnorm(h, self.p("final_norm"), eps)
        z = nf @ self.p("lm_head").T
        lse = logsumexp(z)
        losses = lse - z[np.arange(n), labels]
        saved.update(h_final=h, rf=rf, nf=nf, z=z, lse=lse, labels=labels)
        return losses, saved, new_cache

    def chunk_grad(self, W, saved):
        """Hand-written gradient of A_i(W) = mean chunk loss w.r.t. the fast weights."""
        c = self.cfg
        eps = c.rms_eps  # noqa: F841  (saved r already includes eps)
        z, lse, labels = saved["z"], saved["lse"], saved["labels"]
        n = z.shape[0]
        H, hd = c.n_heads, c.head_dim
        dz = np.exp(z - lse[:, None])
        dz[np.arange(n), labels] -= 1.0
        dz /= n
        dn = dz @ self.p("lm_head")
        dh = rmsnorm_bwd(dn, saved["h_final"], saved["rf"], self.p("final_norm"))
        grads = [None] * self.nu
        cos, sin = saved["cos"], saved["sin"]
        for l in range(self.L - 1, self.first_fast - 1, -1):
            pre = f"l{l}."
            s = saved["layers"][l]
            wg, wu, wd = W[l - self.first_fast]
            G, U, Hm = s["acts_f"]
            m = s["m"]
            # fast SwiGLU branch: y_f = (silu(G) * U) Wd^T
            dWd = dh.T @ Hm
            dHm = dh @ wd
            dG = dHm * U * dsilu(G)
            dU = dHm * silu(G)
            dWg = dG.T @ m
            dWu = dU.T @ m
            grads[l - self.first_fast] = [dWg, dWu, dWd]
            if l == self.first_fast:
                break   # nothing below this MLP depends on W
            # static branch (frozen, but on the path to lower fast weights)
            Gs, Us, _ = s["acts_s"]
            dHs = dh @ self.p(pre + "w_down")
            dGs = dHs * Us * dsilu(Gs)
            dUs = dHs * silu(Gs)
            dm = dG @ wg + dU @ wu + dGs @ self.p(pre + "w_gate") + dUs @ self.p(pre + "w_up")
            dh1 = dh + rmsnorm_bwd(dm, s["h1"], s["r2"], self.p(pre + "mlp_norm"))
            # attention sub-block: h1 = h_in + o Wo^T
            do = (dh1 @ self.p(pre + "wo")).reshape(n, H, hd)
            dqh, dkh, dv = self.attention_bwd(do, s["qh"], s["K"], s["V"], saved["pos"], s["pos_k"], s["n_old"])
            dqn = rope_bwd(dqh, cos, sin)
            dkn = rope_bwd(dkh, cos, sin)
            dq = rmsnorm_bwd(dqn, s["q"], s["rq"], self.p(pre + "q_norm"))
            dk = rmsnorm_bwd(dkn, s["k"], s["rk"], self.p(pre + "k_norm"))
            da = (dq.reshape(n, -1) @ self.p(pre + "wq") + dk.reshape(n, -1) @ self.p(pre + "wk")
                  + dv.reshape(n, -1) @ self.p(pre + "wv"))
            dh = dh1 + rmsnorm_bwd(da, s["h_in"], s["r1"], self.p(pre + "attn_norm"))
        return grads

    # ---------------------------------------------------------------- Algorithm 1
    def prefill(self, tokens, eta=None, no_update=False, W_init=None, return_trace=False, progress=None,
                return_cache=False):
        """Run Algorithm 1 on ids x_0..x_T; returns (losses[T], W_N[, trace]).

        Position p (0 <= p < T) predicts x_{p+1}; chunk i holds positions
        [i*b, min((i+1)*b, T)).  With no_update the SGD step is skipped.
        ``progress(s0, n)``, if given, is called after each chunk (reporting only).
        """
        c = self.cfg
        eta = c.eta if eta is None else eta
        tokens = np.asarray(tokens)
        T = len(tokens) - 1
        b = c.chunk
        W = self.init_fast() if W_init is None else [[w.copy() for w in ws] for ws in W_init]
        cache = self.empty_cache()
        losses = np.zeros(max(T, 0), dtype=self.dt)
        trace = []
        for s0 in range(0, T, b):
            n = min(b, T - s0)
            x_in = tokens[s0:s0 + n]
            labels = tokens[s0 + 1:s0 + n + 1]
            l_chunk, saved, new_cache = self.chunk_forward(W, cache, x_in, labels, s0, consume=not return_trace)
            losses[s0:s0 + n] = l_chunk          # recorded before the update
            if return_trace:
                trace.append({"W_before": [[w.copy() for w in ws] for ws in W],
                              "cache": cache, "s0": s0, "n": n})
            if not no_update and self.nu > 0:
                G = self.chunk_grad(W, saved)
                W = [[sgd_step(w, g, eta) for w, g in zip(ws, gs)] for ws, gs in zip(W, G)]
            cache = new_cache
            if progress is not None:
                progress(s0, n)
        if return_cache:
            return losses, W, cache
        if return_trace:
            return losses, W, trace
        return losses, W

    # ---------------------------------------------------------------- Algorithm 3
    def decode(self, tokens, n_steps, forced=None, eta=None, no_update=False):
        """Generation with periodic updates (the notes, section 7, Algorithm 3) after
        Algorithm 1 on `tokens` = x_0..x_P (P scored positions).

        Positions P, P+1, ... are fed one at a time with the current fast weights and
        attention state; the id after each is forced[j] if given, else the argmax of
        the prediction (lowest id among equal logits).  Decode chunks are
        [P + i*b, P + (i+1)*b) (reading: counted from where the prefill stopped).
        Once a chunk's last target is known, its mean loss under the weights that
        predicted it, with the attention state of the chunk's start, is
        back-propagated and one SGD step taken, exactly as for a prefill chunk,
        before the next position is fed.

        Returns (prefill losses [P], next ids [n_steps], step losses [n_steps],
        top-2 logit margins [n_steps], W).
        """
        c = self.cfg
        eta = c.eta if eta is None else eta
        b = c.chunk
        pre_losses, W, cache = self.prefill(tokens, eta=eta, no_update=no_update, return_cache=True)
        seq = [int(x) for x in np.asarray(tokens)]
        P = len(seq) - 1
        chunk_cache = cache
        s0 = P
        ids = np.zeros(n_steps, dtype=np.int64)
        step_losses = np.zeros(n_steps, dtype=self.dt)
        margins = np.zeros(n_steps, dtype=self.dt)
        for j in range(n_steps):
            p = P + j
            _, saved, cache = self.chunk_forward(W, cache, np.array([seq[p]]), np.array([0]), p)
            z = saved["z"][0]
            nxt = int(forced[j]) if forced is not None else int(np.argmax(z))
            top2 = np.sort(z)[-2:]
            margins[j] = top2[1] - top2[0]
            step_losses[j] = saved["lse"][0] - z[nxt]
            ids[j] = nxt
            seq.append(nxt)
            if p + 1 - s0 == b:
                if not no_update and self.nu > 0:
                    x_in = np.array(seq[s0:s0 + b])
                    labels = np.array(seq[s0 + 1:s0 + b + 1])
                    _, saved_c, cache = self.chunk_forward(W, chunk_cache, x_in, labels, s0)
                    G = self.chunk_grad(W, saved_c)
                    W = [[sgd_step(w, g, eta) for w, g in zip(ws, gs)] for ws, gs in zip(W, G)]
                chunk_cache = cache
                s0 += b
        return pre_losses, ids, step_losses, margins, W

    def chunk_loss(self, W, cache, tokens, s0, n):
        """A_i(W): mean loss of the chunk at [s0, s0+n) with the state `cache` fixed."""
        x_in = np.asarray(tokens[s0:s0 + n])
        labels = np.asarray(tokens[s0 + 1:s0 + n + 1])
        l_chunk, _, _ = self.chunk_forward(W, cache, x_in, labels, s0)
        return float(np.mean(l_chunk))


def prefill(cfg, weights, tokens, dtype=np.float64, **kw):
    """Convenience wrapper: Algorithm 1 on `tokens` with `weights`."""
    return Oracle(cfg, weights, dtype=dtype).prefill(tokens, **kw)

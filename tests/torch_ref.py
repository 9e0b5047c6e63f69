"""Independent whole-sequence reference built from torch library routines.

Used only to pin the oracle: torch's rms_norm, scaled_dot_product_attention,
silu, cross_entropy and autograd stand in for the textbook definitions.  The
rotary embedding is written as a complex rotation (a different formulation
from the oracle's cos/sin form).  No chunking, no cache: the whole sequence is
one forward under an explicit mask, which is what the chunked recurrence must
reproduce when the inner step size is zero (the notes, section 9.2 and
section 5: with one chunk spanning the sequence no scored token sees an update).
"""
import numpy as np
import torch
import torch.nn.functional as F


def _t(a, dt=torch.float64):
    return torch.as_tensor(np.asarray(a), dtype=dt)


def rope_complex(x, pos, theta):
    """x: [T, H, hd]; pairs (i, i+hd/2) as complex numbers rotated by p*theta^(-2i/hd)."""
    hd = x.shape[-1]
    h = hd // 2
    i = torch.arange(h, dtype=torch.float64)
    ang = pos.to(torch.float64)[:, None] * torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * i / hd)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :h], x[..., h:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def forward_losses(cfg, weights, tokens, fast, mask="band", wo_zero=False, return_logits=False):
    """Per-token losses of the whole sequence; `fast` is a list of [wg, wu, wd] tensors.
    With return_logits, the logits [T, V] instead."""
    L, d, H, hd = cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.head_dim
    eps = cfg.rms_eps
    tok = torch.as_tensor(np.asarray(tokens), dtype=torch.long)
    T = len(tok) - 1
    x_in, labels = tok[:T], tok[1:]
    pos = torch.arange(T)
    W = {k: _t(v) for k, v in weights.items() if not k.startswith("fast")}
    h = F.embedding(x_in, W["tok_emb"])
    if mask == "band":
        j = pos[None, :]
        p = pos[:, None]
        attn_mask = (j <= p) & (j > p - cfg.window)
    first_fast = L - cfg.n_update
    for l in range(L):
        pre = f"l{l}."
        a = F.rms_norm(h, (d,), W[pre + "attn_norm"], eps)
        q = F.linear(a, W[pre + "wq"]).view(T, H, hd)
        k = F.linear(a, W[pre + "wk"]).view(T, H, hd)
        v = F.linear(a, W[pre + "wv"]).view(T, H, hd)
        q = rope_complex(F.rms_norm(q, (hd,), W[pre + "q_norm"], eps), pos, cfg.rope_theta)
        k = rope_complex(F.rms_norm(k, (hd,), W[pre + "k_norm"], eps), pos, cfg.rope_theta)
        qT, kT, vT = (t.transpose(0, 1).unsqueeze(0) for t in (q, k, v))
        if mask == "causal":
            o = F.scaled_dot_product_attention(qT, kT, vT, is_causal=True)
        else:
            o = F.scaled_dot_product_attention(qT, kT, vT, attn_mask=attn_mask)
        o = o.squeeze(0).transpose(0, 1).reshape(T, d)
        wo = W[pre + "wo"] * (0.0 if wo_zero else 1.0)
        h = h + F.linear(o, wo)
        m = F.rms_norm(h, (d,), W[pre + "mlp_norm"], eps)
        y = F.linear(F.silu(F.linear(m, W[pre + "w_gate"])) * F.linear(m, W[pre + "w_up"]), W[pre + "w_down"])
        if l >= first_fast:
            wg, wu, wd = fast[l - first_fast]
            y = y + F.linear(F.silu(F.linear(m, wg)) * F.linear(m, wu), wd)
        h = h + y
    n = F.rms_norm(h, (d,), W["final_norm"], eps)
    z = F.linear(n, W["lm_head"])
    if return_logits:
        return z
    return F.cross_entropy(z, labels, reduction="none")


def fast_tensors(fast_np, requires_grad=False):
    return [[_t(w).requires_grad_(requires_grad) for w in ws] for ws in fast_np]


def fast_from_weights(cfg, weights):
    return [[weights[f"fast{u}.w_gate"], weights[f"fast{u}.w_up"], weights[f"fast{u}.w_down"]]
            for u in range(cfg.n_update)]

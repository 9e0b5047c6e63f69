"""Seeded synthetic weights, bit-identical on the host (numpy) and on a device (torch).

The pages never give an initialisation; the workloads use a zero-mean draw with
standard deviation 0.02 for every matrix and unit gains for every norm.  To get
exactly the same values from numpy on the host and from torch on a GPU, each
element is produced by a counter-based generator rather than a stateful stream:

  key_t      = splitmix64(seed * 0x100000001B3 + tensor_id)
  x          = splitmix64(key_t + flat_index)              (uint64, wrapping)
  s          = sum of the four 16-bit fields of x  - 131070  (an integer)
  value      = float32(s) * C,   C = float32(std / sqrt(4 * (65536**2 - 1) / 12))

so a value is a scaled sum of four independent uniform 16-bit integers (an
Irwin-Hall approximation of a normal law with the requested mean and standard
deviation, tails cut at about 3.46 sigma).  Every step is integer arithmetic
except one IEEE float32 multiply, which rounds identically everywhere.  bf16
workloads then round to nearest-even bf16.  splitmix64 is Steele, Lea and
Flood's SplitMix finaliser (OOPSLA 2014), with Vigna's published constants.

This module holds no arithmetic of the method itself.
"""
import math
import numpy as np

_GOLD = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_U64 = (1 << 64) - 1


def _splitmix64_scalar(x):
    z = (x + _GOLD) & _U64
    z = ((z ^ (z >> 30)) * _M1) & _U64
    z = ((z ^ (z >> 27)) * _M2) & _U64
    return z ^ (z >> 31)


def tensor_key(seed, tensor_id):
    return _splitmix64_scalar((seed * 0x100000001B3 + tensor_id) & _U64)


def scale_const(std):
    return np.float32(std / math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0))


# ---------------------------------------------------------------- numpy side
def _np_values(key, start, count, c32):
    with np.errstate(over="ignore"):
        x = np.arange(start, start + count, dtype=np.uint64) + np.uint64(key)
        z = x + np.uint64(_GOLD)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    m = np.uint64(0xFFFF)
    s = ((z & m) + ((z >> np.uint64(16)) & m) + ((z >> np.uint64(32)) & m)
         + (z >> np.uint64(48))).astype(np.int64) - 131070
    return s.astype(np.float32) * c32


def round_bf16_np(a):
    """Round float32 values to nearest-even bf16, returned as float32."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def draw_np(seed, tensor_id, shape, std, bf16, block=1 << 24):
    n = int(np.prod(shape))
    key = tensor_key(seed, tensor_id)
    c32 = scale_const(std)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, block):
        cnt = min(block, n - s)
        out[s:s + cnt] = _np_values(key, s, cnt, c32)
    if bf16:
        out = round_bf16_np(out)
    return out.reshape(shape)


# ---------------------------------------------------------------- torch side
def _i64(u):
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(t, n):
    return (t >> n) & ((1 << (64 - n)) - 1)


def draw_torch(seed, tensor_id, shape, std, bf16, device, block=1 << 26):
    import torch
    n = int(np.prod(shape))
    key = tensor_key(seed, tensor_id)
    c32 = float(scale_const(std))
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, block):
        cnt = min(block, n - s)
        x = torch.arange(s, s + cnt, dtype=torch.int64, device=device)
        z = x + _i64((key + _GOLD) & _U64)
        z = (z ^ _lsr(z, 30)) * _i64(_M1)
        z = (z ^ _lsr(z, 27)) * _i64(_M2)
        z = z ^ _lsr(z, 31)
        s16 = (z & 0xFFFF) + (_lsr(z, 16) & 0xFFFF) + (_lsr(z, 32) & 0xFFFF) + _lsr(z, 48)
        out[s:s + cnt] = (s16 - 131070).to(torch.float32) * c32
    out = out.reshape(shape)
    if bf16:
        out = out.to(torch.bfloat16)
    return out


# ---------------------------------------------------------------- model layout
def tensor_specs(cfg):
    """(name, tensor_id, shape, kind) for every weight; kind in {mat, gain, fast}."""
    d, F, V, hd = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.head_dim
    specs = [("tok_emb", 0, (V, d), "mat"), ("lm_head", 1, (V, d), "mat"),
             ("final_norm", 2, (d,), "gain")]
    for l in range(cfg.n_layers):
        b = 16 + 8 * l
        specs += [(f"l{l}.attn_norm", None, (d,), "gain"),
                  (f"l{l}.wq", b + 0, (d, d), "mat"), (f"l{l}.wk", b + 1, (d, d), "mat"),
                  (f"l{l}.wv", b + 2, (d, d), "mat"), (f"l{l}.wo", b + 3, (d, d), "mat"),
                  (f"l{l}.q_norm", None, (hd,), "gain"), (f"l{l}.k_norm", None, (hd,), "gain"),
                  (f"l{l}.mlp_norm", None, (d,), "gain"),
                  (f"l{l}.w_gate", b + 4, (F, d), "mat"), (f"l{l}.w_up", b + 5, (F, d), "mat"),
                  (f"l{l}.w_down", b + 6, (d, F), "mat")]
    for u in range(cfg.n_update):
        b = 1_000_000 + 4 * u
        specs += [(f"fast{u}.w_gate", b + 0, (F, d), "fast"),
                  (f"fast{u}.w_up", b + 1, (F, d), "fast"),
                  (f"fast{u}.w_down", b + 2, (d, F), "fast")]
    return specs


def random_gains(cfg, seed, norm_range=(0.5, 1.5), qk_range=None):
    """Non-unit norm gains for tests: each gain vector (block norms, final norm, QK-norm)
    drawn uniform in its range from its own PCG64 stream seeded by (seed, position in
    tensor_specs), rounded to bf16 so that bf16 and fp32 workloads hold the same values.
    qk_range (default: norm_range) applies to q_norm and k_norm."""
    qk_range = norm_range if qk_range is None else qk_range
    out = {}
    for i, (name, _, shape, kind) in enumerate(tensor_specs(cfg)):
        if kind != "gain":
            continue
        lo, hi = qk_range if name.endswith(("q_norm", "k_norm")) else norm_range
        g = np.random.Generator(np.random.PCG64([seed, i])).uniform(lo, hi, shape).astype(np.float32)
        out[name] = round_bf16_np(g)
    return out


def make_weights_np(cfg, seed=0, names=None, gains=None):
    """All weights as float32 numpy arrays (bf16-valued for bf16 workloads).  gains:
    None for unit norm gains, or a dict from random_gains replacing them."""
    bf16 = cfg.dtype == "bf16"
    out = {}
    for name, tid, shape, kind in tensor_specs(cfg):
        if names is not None and name not in names:
            continue
        if kind == "gain":
            out[name] = gains[name].copy() if gains is not None else np.ones(shape, dtype=np.float32)
        else:
            out[name] = draw_np(seed, tid, shape, cfg.init_std, bf16)
    return out


def make_weights_torch(cfg, device, seed=0, gains=None):
    """Weights as torch tensors on `device`: the working dtype for frozen tensors,
    float32 (bf16-valued in bf16 workloads) for the fast-weight initial values.
    gains as for make_weights_np."""
    import torch
    bf16 = cfg.dtype == "bf16"
    wdt = torch.bfloat16 if bf16 else torch.float32
    out = {}
    for name, tid, shape, kind in tensor_specs(cfg):
        if kind == "gain":
            if gains is not None:
                out[name] = torch.from_numpy(gains[name]).to(device=device, dtype=wdt)
            else:
                out[name] = torch.ones(shape, dtype=wdt, device=device)
        elif kind == "fast":
            out[name] = draw_torch(seed, tid, shape, cfg.init_std, bf16, device).to(torch.float32)
        else:
            out[name] = draw_torch(seed, tid, shape, cfg.init_std, bf16, device).to(wdt)
    return out

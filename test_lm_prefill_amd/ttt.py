"""ctypes binding of libttt.so (the C ABI in include/ttt.h).

Argument marshalling only: every step of the prefill runs in the library's
HIP kernels.  torch is used for device memory and the current stream.  If the
built library is missing this module raises at import of the first call; there
is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt.so")

TTT_OK, TTT_EINVAL, TTT_ENOMEM, TTT_EHIP, TTT_EUNSUPPORTED, TTT_ENONFINITE = 0, -1, -2, -3, -4, -5
TTT_FP32, TTT_BF16 = 0, 1
TTT_NO_UPDATE, TTT_NO_GRAPH = 1, 2

EXPORTED = ["ttt_create", "ttt_prefill", "ttt_prefill_noalloc", "ttt_decode", "ttt_check_finite", "ttt_get_stats", "ttt_set_kernel_timing",
            "ttt_kernel_class_count", "ttt_get_kernel_time", "ttt_last_error", "ttt_destroy"]


class ttt_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("window", ctypes.c_int32), ("chunk", ctypes.c_int32), ("n_update", ctypes.c_int32),
                ("eta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("max_tokens", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("n_seq", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class ttt_weights(ctypes.Structure):
    _fields_ = [("tok_emb", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP),
                ("q_norm", _PP), ("k_norm", _PP), ("mlp_norm", _PP),
                ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP),
                ("fast_gate", _PP), ("fast_up", _PP), ("fast_down", _PP)]


class TTTError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("ttt status %d: %s" % (status, msg))
        self.status = status


_lib = None


def lib():
    """Loads libttt.so (built by test_lm_prefill_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libttt.so is not built; run `python -m test_lm_prefill_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.ttt_create.argtypes = [ctypes.POINTER(ttt_config), ctypes.POINTER(ttt_weights), ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_void_p)]
        L.ttt_create.restype = ctypes.c_int
        L.ttt_prefill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, _PP,
                                  ctypes.c_uint32, ctypes.c_void_p]
        L.ttt_prefill.restype = ctypes.c_int
        L.ttt_prefill_noalloc.argtypes = L.ttt_prefill.argtypes
        L.ttt_prefill_noalloc.restype = ctypes.c_int
        L.ttt_decode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 _PP, ctypes.c_uint32, ctypes.c_void_p]
        L.ttt_decode.restype = ctypes.c_int
        L.ttt_check_finite.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.ttt_check_finite.restype = ctypes.c_int
        L.ttt_get_stats.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64)]
        L.ttt_get_stats.restype = ctypes.c_int
        L.ttt_set_kernel_timing.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.ttt_set_kernel_timing.restype = ctypes.c_int
        L.ttt_kernel_class_count.argtypes = []
        L.ttt_kernel_class_count.restype = ctypes.c_int
        L.ttt_get_kernel_time.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.ttt_get_kernel_time.restype = ctypes.c_int
        L.ttt_last_error.argtypes = [ctypes.c_void_p]
        L.ttt_last_error.restype = ctypes.c_char_p
        L.ttt_destroy.argtypes = [ctypes.c_void_p]
        L.ttt_destroy.restype = None
        _lib = L
    return _lib


def _check(status, handle=None):
    if status != TTT_OK:
        msg = lib().ttt_last_error(handle)
        raise TTTError(status, msg.decode() if msg else "")


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return ctypes.cast(arr, _PP), arr


# ---------------------------------------------------------------- same-name entry points
def ttt_create(cfg, weights, stream=None):
    """cfg: ttt_config; weights: ttt_weights; stream: hipStream_t as int or None. Returns the handle."""
    h = ctypes.c_void_p()
    st = lib().ttt_create(ctypes.byref(cfg), ctypes.byref(weights), stream, ctypes.byref(h))
    _check(st)
    return h.value


def ttt_prefill(handle, d_tokens, T, d_losses, d_fast_out=None, flags=0, stream=None):
    fo = None
    keep = None
    if d_fast_out is not None:
        fo, keep = _ptr_array(d_fast_out)
    st = lib().ttt_prefill(handle, d_tokens, T, d_losses, fo, flags, stream)
    del keep
    _check(st, handle)


def ttt_prefill_noalloc(handle, d_tokens, T, d_losses, d_fast_out=None, flags=0, stream=None):
    fo = None
    keep = None
    if d_fast_out is not None:
        fo, keep = _ptr_array(d_fast_out)
    st = lib().ttt_prefill_noalloc(handle, d_tokens, T, d_losses, fo, flags, stream)
    del keep
    _check(st, handle)


def ttt_decode(handle, n_steps, d_forced, d_tokens_out, d_losses_out, d_fast_out=None, flags=0, stream=None):
    fo = None
    keep = None
    if d_fast_out is not None:
        fo, keep = _ptr_array(d_fast_out)
    st = lib().ttt_decode(handle, n_steps, d_forced, d_tokens_out, d_losses_out, fo, flags, stream)
    del keep
    _check(st, handle)


def ttt_check_finite(handle, stream=None):
    _check(lib().ttt_check_finite(handle, stream), handle)


def ttt_get_stats(handle):
    """Returns (ms of the last prefill, its chunks, kernel launches per chunk step)."""
    ms, a, b = ctypes.c_double(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ttt_get_stats(handle, ctypes.byref(ms), ctypes.byref(a), ctypes.byref(b)), handle)
    return ms.value, a.value, b.value


def ttt_set_kernel_timing(handle, enable):
    _check(lib().ttt_set_kernel_timing(handle, 1 if enable else 0), handle)


def ttt_kernel_class_count():
    return lib().ttt_kernel_class_count()


def ttt_get_kernel_time(handle, cls):
    """Returns (name, total_ms, launches) of kernel class `cls`."""
    nm, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
    _check(lib().ttt_get_kernel_time(handle, cls, ctypes.byref(nm), ctypes.byref(ms), ctypes.byref(n)), handle)
    return nm.value.decode(), ms.value, n.value


def ttt_last_error(handle=None):
    m = lib().ttt_last_error(handle)
    return m.decode() if m else ""


def ttt_destroy(handle):
    lib().ttt_destroy(handle)


# ---------------------------------------------------------------- convenience session
class Session:
    """Holds one handle built from a dict of device tensors named as in the
    workload generators (tok_emb, lm_head, final_norm, l{i}.wq, ..., fast{u}.w_gate, ...)."""

    def __init__(self, cfg, weights, max_tokens=None, flags=0, n_seq=1):
        import torch
        self.torch = torch
        self.cfg = cfg
        c = ttt_config()
        c.n_layers, c.d_model, c.n_heads = cfg.n_layers, cfg.d_model, cfg.n_heads
        c.head_dim, c.d_ff, c.vocab = cfg.head_dim, cfg.d_ff, cfg.vocab
        c.window, c.chunk, c.n_update = cfg.window, cfg.chunk, cfg.n_update
        c.eta, c.rms_eps, c.rope_theta = cfg.eta, cfg.rms_eps, cfg.rope_theta
        c.dtype = TTT_BF16 if cfg.dtype == "bf16" else TTT_FP32
        c.max_tokens = int(max_tokens if max_tokens is not None else cfg.seq_len)
        c.flags = flags
        c.n_seq = int(n_seq)
        self.n_seq = max(1, int(n_seq))
        self.c = c
        L, nu = cfg.n_layers, cfg.n_update
        w = ttt_weights()
        keep = []

        def ptr(name):
            t = weights[name]
            assert t.is_cuda and t.is_contiguous(), name
            return t.data_ptr()

        def arr(fmt, n):
            p, a = _ptr_array([ptr(fmt.format(i)) for i in range(n)])
            keep.append(a)
            return p

        w.tok_emb, w.lm_head, w.final_norm = ptr("tok_emb"), ptr("lm_head"), ptr("final_norm")
        for f, nm in [("attn_norm", "attn_norm"), ("wq", "wq"), ("wk", "wk"), ("wv", "wv"), ("wo", "wo"),
                      ("q_norm", "q_norm"), ("k_norm", "k_norm"), ("mlp_norm", "mlp_norm"),
                      ("w_gate", "w_gate"), ("w_up", "w_up"), ("w_down", "w_down")]:
            setattr(w, f, arr("l{}." + nm, L))
        for f, nm in [("fast_gate", "w_gate"), ("fast_up", "w_up"), ("fast_down", "w_down")]:
            setattr(w, f, arr("fast{}." + nm, nu) if nu > 0 else None)
        self._keep = keep
        stream = torch.cuda.current_stream().cuda_stream
        self.handle = ttt_create(c, w, stream)

    def prefill(self, tokens, flags=0, want_fast=True, check=True):
        """tokens: int32 device tensor [T+1] (one sequence) or [B, T+1] (B = n_seq).
        Returns (losses [T] or [B, T] fp32, fast tensors or None: a flat list of 3*n_u
        for one sequence, a list of B such lists otherwise)."""
        torch = self.torch
        assert tokens.dtype == torch.int32 and tokens.is_cuda and tokens.is_contiguous()
        batched = tokens.dim() == 2
        B = tokens.shape[0] if batched else 1
        assert B == self.n_seq, "the token batch must hold n_seq sequences"
        T = tokens.shape[-1] - 1
        dev = tokens.device
        losses = torch.empty((B, max(T, 0)) if batched else (max(T, 0),), dtype=torch.float32, device=dev)
        fast = None
        ptrs = None
        if want_fast and self.cfg.n_update > 0:
            fast = [self._fast_buffers(dev) for _ in range(B)]
            ptrs = [t.data_ptr() for fs in fast for t in fs]
        stream = torch.cuda.current_stream().cuda_stream
        ttt_prefill(self.handle, tokens.data_ptr(), T, losses.data_ptr() if T > 0 else None, ptrs, flags, stream)
        if check:
            ttt_check_finite(self.handle, stream)
        if fast is not None and not batched:
            fast = fast[0]
        return losses, fast

    def _fast_buffers(self, dev):
        torch = self.torch
        F, d = self.cfg.d_ff, self.cfg.d_model
        fast = []
        for _ in range(self.cfg.n_update):
            fast += [torch.empty(F, d, dtype=torch.float32, device=dev),
                     torch.empty(F, d, dtype=torch.float32, device=dev),
                     torch.empty(d, F, dtype=torch.float32, device=dev)]
        return fast

    def decode(self, n_steps, forced=None, flags=0, want_fast=True, check=True):
        """Continues the last prefill (Algorithm 3).  forced: int32 device tensor [n_steps]
        of next ids, or None for greedy.  Returns (next ids [n_steps] int32, losses
        [n_steps] fp32, fast tensors or None)."""
        torch = self.torch
        dev = torch.device("cuda", torch.cuda.current_device())
        if forced is not None:
            assert forced.dtype == torch.int32 and forced.is_cuda and forced.is_contiguous()
            assert forced.numel() == n_steps
        toks = torch.empty(max(n_steps, 0), dtype=torch.int32, device=dev)
        losses = torch.empty(max(n_steps, 0), dtype=torch.float32, device=dev)
        fast = self._fast_buffers(dev) if want_fast and self.cfg.n_update > 0 else None
        ptrs = [t.data_ptr() for t in fast] if fast is not None else None
        stream = torch.cuda.current_stream().cuda_stream
        ttt_decode(self.handle, n_steps, forced.data_ptr() if forced is not None else None,
                   toks.data_ptr() if n_steps > 0 else None, losses.data_ptr() if n_steps > 0 else None,
                   ptrs, flags, stream)
        if check:
            ttt_check_finite(self.handle, stream)
        return toks, losses, fast

    def stats(self):
        return ttt_get_stats(self.handle)

    def kernel_times(self):
        """{class name: (total ms, launches)} collected while kernel timing was on."""
        out = {}
        for c in range(ttt_kernel_class_count()):
            nm, ms, n = ttt_get_kernel_time(self.handle, c)
            out[nm] = (ms, n)
        return out

    def set_kernel_timing(self, enable):
        ttt_set_kernel_timing(self.handle, enable)

    def close(self):
        if self.handle:
            ttt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

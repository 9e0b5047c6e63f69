"""The C-ABI library loads and exports every entry point include/ttt.h declares (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(ttt_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["ttt_create", "ttt_prefill", "ttt_check_finite", "ttt_get_stats", "ttt_last_error", "ttt_destroy"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    from test_lm_prefill_amd import ttt
    if not os.path.exists(ttt.LIB_PATH):
        pytest.skip("libttt.so not built")
    lib = ctypes.CDLL(ttt.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(ttt.EXPORTED) == set(declared_functions())


def test_create_rejects_bad_config_without_gpu_work():
    """Validation happens before any device call, so it runs on the CPU."""
    from test_lm_prefill_amd import ttt
    if not os.path.exists(ttt.LIB_PATH):
        pytest.skip("libttt.so not built")
    c = ttt.ttt_config()
    c.n_layers, c.d_model, c.n_heads, c.head_dim = 2, 64, 4, 17   # d != H*hd
    c.d_ff, c.vocab, c.window, c.chunk, c.n_update = 256, 256, 256, 128, 1
    c.eta, c.rms_eps, c.rope_theta, c.dtype, c.max_tokens = 0.1, 1e-6, 1e4, 0, 2048
    w = ttt.ttt_weights()
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_create(c, w)
    assert e.value.status == ttt.TTT_EINVAL
    c.head_dim = 16
    c.chunk = 100      # not a multiple of 64
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_create(c, w)
    assert e.value.status == ttt.TTT_EINVAL
    c.chunk, c.window = 128, 64   # window < chunk
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_create(c, w)
    assert e.value.status == ttt.TTT_EINVAL
    c.window = 256
    with pytest.raises(ttt.TTTError) as e:     # null weights
        ttt.ttt_create(c, w)
    assert e.value.status == ttt.TTT_EINVAL
    assert "null" in ttt.ttt_last_error()

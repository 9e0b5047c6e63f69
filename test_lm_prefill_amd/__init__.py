"""MI355X-native TTT-E2E prefill: libttt.so (HIP, gfx950) and its ctypes binding."""
from .ttt import Session, lib  # noqa: F401

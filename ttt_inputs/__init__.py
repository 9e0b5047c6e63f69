"""Seeded synthetic inputs (configs, weights, tokens) for the TTT-E2E prefill.

Serves both the CPU oracle and the GPU library's callers; holds none of the
method's arithmetic.
"""
from .configs import TTTConfig, CONFIGS, get  # noqa: F401
from .weights import make_weights_np, make_weights_torch, tensor_specs, round_bf16_np, random_gains  # noqa: F401
from .tokens import make_tokens, markov2_tokens, zipf_span_tokens  # noqa: F401

"""Model and run shapes for the TTT-E2E prefill workloads.

These are data, shared by the CPU oracle and the GPU library's callers.  The
model families follow the sizes listed on the jdon.com page (the "basic recipe"
paragraph: 125M 12x768x12 ... 2.7B 32x2560x32); the window k=8K, chunk b=1K and
"last quarter of blocks updated" choice follow the zhongzhuzhou.org notes
(section 5 and section 6) and the jdon.com ablation paragraph.  The SwiGLU
hidden sizes, RMSNorm, RoPE, the inner learning rate and the precisions are not
on the pages; they are fixed here.
"""
from dataclasses import dataclass, asdict, replace


@dataclass(frozen=True)
class TTTConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    seq_len: int          # T: number of scored positions (T+1 token ids)
    window: int           # k: sliding attention window
    chunk: int            # b: tokens per inner update
    n_update: int         # n_u: number of trailing blocks with fast MLPs
    eta: float            # inner SGD step size
    dtype: str            # "fp32" or "bf16"
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    init_std: float = 0.02
    tokens: str = "zipf_span"   # or "markov2"

    def as_dict(self):
        return asdict(self)

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def n_chunks(self):
        return -(-self.seq_len // self.chunk)


TINY = TTTConfig("tiny", 2, 64, 4, 16, 256, 256, 2048, 256, 128, 1, 0.1, "fp32",
                 tokens="markov2")
M125 = TTTConfig("125m", 12, 768, 12, 64, 2048, 128256, 32768, 8192, 1024, 3, 0.01, "bf16")
M760 = TTTConfig("760m", 24, 1536, 16, 96, 4096, 128256, 131072, 8192, 1024, 6, 0.01, "bf16")
B13_256 = TTTConfig("1.3b_b256", 24, 2048, 32, 64, 5504, 128256, 65536, 8192, 256, 6, 0.01, "bf16")
B13_1K = B13_256.with_(name="1.3b_b1024", chunk=1024)
B13_4K = B13_256.with_(name="1.3b_b4096", chunk=4096)
B27_8K = TTTConfig("2.7b_8k", 32, 2560, 32, 80, 6912, 128256, 8192, 8192, 1024, 8, 0.01, "bf16")
B27_32K = B27_8K.with_(name="2.7b_32k", seq_len=32768)
B27_128K = B27_8K.with_(name="2.7b_128k", seq_len=131072)

CONFIGS = {c.name: c for c in [TINY, M125, M760, B13_256, B13_1K, B13_4K,
                               B27_8K, B27_32K, B27_128K]}


def get(name):
    return CONFIGS[name]

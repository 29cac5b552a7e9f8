"""Workload shapes.

The three layer shapes follow the public configurations of the models the Collider paper evaluates
("Enhancing Token Filtering Efficiency in Large Language Model Training with Collider", abstract:
TinyLlama-1.1B, Qwen2.5-1.5B and Phi1.5-1.4B).  The filter ratio of 40% is the one the abstract's
headline figures are quoted at; the Figure 4 caption gives 30-40% as the typical range.
The paper's training data and weights are not used: every tensor is drawn from a seed.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LinearShape:
    """A single linear layer y = x @ w.T with x [M, K], w [N, K], trained in fp32."""
    name: str
    B: int
    S: int
    K: int
    N: int
    r_pct: int = 40
    seed: int = 0
    kind: str = "linear"

    @property
    def M(self) -> int:
        return self.B * self.S


@dataclass(frozen=True)
class LayerShape:
    """One pre-norm decoder layer.

    kind "llama": x -> RMSNorm -> QKV (+RoPE) -> causal GQA attention -> O, residual,
                  RMSNorm -> gate/up -> SwiGLU -> down, residual.
    kind "phi":   parallel block: LayerNorm once, attention and GELU-tanh MLP both read it,
                  y = x + attn + mlp.
    No projection biases.
    """
    name: str
    kind: str
    B: int
    S: int
    H: int
    nq: int
    nkv: int
    d: int
    I: int
    rot: int
    rope_base: float
    eps: float
    r_pct: int = 40
    seed: int = 0
    n_layers: int = 1

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def n_qkv(self) -> int:
        return (self.nq + 2 * self.nkv) * self.d

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


CONFIGS = {
    # fp32 single linear layer, 256x256, 40% filtered (154 of 256 rows kept)
    "linear_fp32": LinearShape("linear_fp32", B=1, S=256, K=256, N=256),
    # TinyLlama-1.1B-shaped layer, batch 4 x seq 2048
    "tinyllama": LayerShape("tinyllama", "llama", B=4, S=2048, H=2048, nq=32, nkv=4, d=64,
                            I=5632, rot=64, rope_base=1.0e4, eps=1e-5),
    # Qwen2.5-1.5B-shaped layer, batch 2 x seq 4096
    "qwen25": LayerShape("qwen25", "llama", B=2, S=4096, H=1536, nq=12, nkv=2, d=128,
                         I=8960, rot=128, rope_base=1.0e6, eps=1e-6),
    # Phi-1.5-shaped layer (parallel block, partial rotary 32 of 64), batch 4 x seq 2048
    "phi15": LayerShape("phi15", "phi", B=4, S=2048, H=2048, nq=32, nkv=32, d=64,
                        I=8192, rot=32, rope_base=1.0e4, eps=1e-5),
    # 22 TinyLlama-shaped layers at batch 1 x seq 8192
    "tinyllama_22l": LayerShape("tinyllama_22l", "llama", B=1, S=8192, H=2048, nq=32, nkv=4,
                                d=64, I=5632, rot=64, rope_base=1.0e4, eps=1e-5, n_layers=22),
    # Long-context attention check: one sequence of 16384 tokens with few heads (the kernels' work
    # per sequence grows with S; the head count only multiplies it), small hidden size
    "longctx_attn": LayerShape("longctx_attn", "llama", B=1, S=16384, H=256, nq=4, nkv=1, d=64,
                               I=256, rot=64, rope_base=1.0e4, eps=1e-5),
    # Small shapes that still span several GEMM / attention tiles and a ragged tail.
    "small_llama": LayerShape("small_llama", "llama", B=2, S=200, H=256, nq=4, nkv=2, d=64,
                              I=384, rot=64, rope_base=1.0e4, eps=1e-5),
    "small_llama_d128": LayerShape("small_llama_d128", "llama", B=2, S=176, H=256, nq=4, nkv=2,
                                   d=128, I=512, rot=128, rope_base=1.0e6, eps=1e-6),
    "small_phi": LayerShape("small_phi", "phi", B=2, S=200, H=256, nq=4, nkv=4, d=64, I=512,
                            rot=32, rope_base=1.0e4, eps=1e-5),
}


def get_config(name: str):
    return CONFIGS[name]

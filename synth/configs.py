"""Workload shapes for the Q8_0 prefill forward.

Each ``ModelConfig`` is one decoder shape plus one prompt.  The shapes follow the
Qwen2 layer written out node by node on the page "05 - Graph build - the IR and
the builder" (section 2.5: hidden 896, 14 query heads of dim 64, 2 KV heads, FFN
4864, vocabulary 151936 for the 0.5B model) and scale up to the 7B/8B shapes.

This module holds no arithmetic of the method: only sizes, flags and seeds.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_head: int
    n_head_kv: int
    head_dim: int
    ffn: int
    vocab: int
    n_tokens: int          # tokens in the timed call
    n_ctx: int             # KV region rows per layer
    seed: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    qkv_bias: bool = True  # Qwen2 family carries Q/K/V biases
    qk_norm: bool = False  # Qwen3 per-head RMSNorm on Q and K
    tied: bool = False     # lm_head shares token_embd
    prefix_tokens: int = 0  # tokens prefilled (untimed) before the timed chunk
    description: str = ""

    @property
    def n_embd_q(self) -> int:
        return self.n_head * self.head_dim

    @property
    def n_kv_embd(self) -> int:
        return self.n_head_kv * self.head_dim

    @property
    def first_pos(self) -> int:
        return self.prefix_tokens

    def kv_bytes_per_token(self) -> int:
        """f32 K and V rows over all layers (bytes per context slot)."""
        return 2 * self.n_kv_embd * 4 * self.n_layers

    def with_(self, **kw) -> "ModelConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return ModelConfig(**d)


LAYER1 = ModelConfig(
    name="layer1_896", n_layers=1, hidden=896, n_head=14, n_head_kv=2, head_dim=64,
    ffn=4864, vocab=8192, n_tokens=16, n_ctx=64, seed=0, qkv_bias=True, tied=False,
    description="one Qwen2-0.5B-shaped decoder layer then lm_head (vocab 8192), 16 tokens at 0..15, n_ctx 64",
)

QWEN2_0P5B = ModelConfig(
    name="qwen2_0p5b_pp512", n_layers=24, hidden=896, n_head=14, n_head_kv=2, head_dim=64,
    ffn=4864, vocab=151936, n_tokens=512, n_ctx=4096, seed=2, qkv_bias=True, tied=True,
    description="24-layer Qwen2-0.5B shape, tied Q8_0 embeddings, 512-token prompt at 0..511, n_ctx 4096",
)

QWEN2P5_7B = ModelConfig(
    name="qwen2p5_7b_pp2048", n_layers=28, hidden=3584, n_head=28, n_head_kv=4, head_dim=128,
    ffn=18944, vocab=152064, n_tokens=2048, n_ctx=4096, seed=3, qkv_bias=True, tied=False,
    description="28-layer Qwen2.5-7B shape with QKV bias, 2048-token prompt at 0..2047, n_ctx 4096",
)

QWEN3_8B = ModelConfig(
    name="qwen3_8b_chunk3072at1024", n_layers=36, hidden=4096, n_head=32, n_head_kv=8, head_dim=128,
    ffn=12288, vocab=151936, n_tokens=3072, n_ctx=4096, seed=4, qkv_bias=False, qk_norm=True,
    tied=False, prefix_tokens=1024,
    description="36-layer Qwen3-8B shape with per-head QK RMSNorm; 3072-token chunk at 1024..4095 "
                "over a KV cache prefilled from a 1024-token prefix, n_ctx 4096",
)

MODEL_CONFIGS = {c.name: c for c in (LAYER1, QWEN2_0P5B, QWEN2P5_7B, QWEN3_8B)}


@dataclass(frozen=True)
class GemmCase:
    m: int  # tokens
    k: int
    n: int
    seed: int = 1
    outlier_frac: float = 0.01
    outlier_scale: float = 20.0

    @property
    def name(self) -> str:
        return f"gemm_m{self.m}_k{self.k}_n{self.n}"


GEMM_SWEEP = (
    GemmCase(512, 3584, 3584),
    GemmCase(512, 3584, 18944),
    GemmCase(512, 18944, 3584),
    GemmCase(2048, 4096, 12288),
)

# The configuration the prefill tokens/s headline is quoted on.
HEADLINE = QWEN2_0P5B

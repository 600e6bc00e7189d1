"""Seeded synthetic inputs shared by the oracle and the GPU path.

Nothing here performs any step of the prefill method (no quantization, no
normalisation, no matmul): it only draws numbers.

Recipe (one independent stream per tensor, so any tensor can be regenerated
alone, in any order, on any device):

* matmul weights (token_embd, attn_q/k/v/output, ffn_gate/up/down, output):
  f32 draws of N(0, 0.02^2), laid out row-major [out][in] as GGUF stores them;
* norm gains (attn_norm, ffn_norm, output_norm, attn_q_norm, attn_k_norm):
  1 + N(0, 0.02^2) in f32;
* Q/K/V biases: N(0, 0.02^2) in f32;
* token ids: uniform integers in [0, vocab);
* GEMM-sweep activations: N(0, 1) f32, each element independently scaled by 20
  with probability 0.01 (outliers).

Streams: ``torch.Generator(device).manual_seed(stream_seed(seed, name))`` for
float tensors (so the large weight sets are drawn where they are used; the
stream differs between a CPU and a GPU generator, so a comparison always draws
once and hands the same tensor to both sides), and numpy PCG64 for token ids
(device independent).
"""
from __future__ import annotations

import zlib
from typing import Iterator

import numpy as np
import torch

from .configs import GemmCase, ModelConfig

WEIGHT_STD = 0.02


def stream_seed(seed: int, name: str) -> int:
    """64-bit seed of the stream that draws tensor ``name`` of workload ``seed``."""
    h = (seed * 0x9E3779B97F4A7C15 + zlib.crc32(name.encode())) & ((1 << 63) - 1)
    return h


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, name))
    return g


def tensor_specs(cfg: ModelConfig):
    """(name, shape, kind) for every tensor of the model, in GGUF naming.

    kind is "q8" (a matmul weight, stored quantized), "norm" (an RMSNorm gain)
    or "bias" (a Q/K/V bias).  Shapes are memory shapes: [out][in] for weights.
    """
    h, q, kv, f = cfg.hidden, cfg.n_embd_q, cfg.n_kv_embd, cfg.ffn
    specs = [("token_embd.weight", (cfg.vocab, h), "q8")]
    for i in range(cfg.n_layers):
        p = f"blk.{i}."
        specs.append((p + "attn_norm.weight", (h,), "norm"))
        specs.append((p + "attn_q.weight", (q, h), "q8"))
        specs.append((p + "attn_k.weight", (kv, h), "q8"))
        specs.append((p + "attn_v.weight", (kv, h), "q8"))
        if cfg.qkv_bias:
            specs.append((p + "attn_q.bias", (q,), "bias"))
            specs.append((p + "attn_k.bias", (kv,), "bias"))
            specs.append((p + "attn_v.bias", (kv,), "bias"))
        if cfg.qk_norm:
            specs.append((p + "attn_q_norm.weight", (cfg.head_dim,), "norm"))
            specs.append((p + "attn_k_norm.weight", (cfg.head_dim,), "norm"))
        specs.append((p + "attn_output.weight", (h, q), "q8"))
        specs.append((p + "ffn_norm.weight", (h,), "norm"))
        specs.append((p + "ffn_gate.weight", (f, h), "q8"))
        specs.append((p + "ffn_up.weight", (f, h), "q8"))
        specs.append((p + "ffn_down.weight", (h, f), "q8"))
    specs.append(("output_norm.weight", (h,), "norm"))
    if not cfg.tied:
        specs.append(("output.weight", (cfg.vocab, h), "q8"))
    return specs


def gen_tensor(cfg_seed: int, name: str, shape, kind: str, device="cpu") -> torch.Tensor:
    """Draw one f32 tensor of the model deterministically from its own stream."""
    g = _gen(cfg_seed, name, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(WEIGHT_STD)
    if kind == "norm":
        t.add_(1.0)
    return t


def iter_tensors(cfg: ModelConfig, device="cpu") -> Iterator[tuple[str, str, torch.Tensor]]:
    for name, shape, kind in tensor_specs(cfg):
        yield name, kind, gen_tensor(cfg.seed, name, shape, kind, device)


def gen_token_ids(cfg: ModelConfig) -> tuple[np.ndarray, np.ndarray]:
    """(prefix_ids, chunk_ids) as int32; prefix is empty unless cfg.prefix_tokens > 0."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        cfg.seed, spawn_key=(zlib.crc32(b"token_ids"),))))
    ids = rng.integers(0, cfg.vocab, size=cfg.prefix_tokens + cfg.n_tokens, dtype=np.int64)
    ids = ids.astype(np.int32)
    return ids[: cfg.prefix_tokens].copy(), ids[cfg.prefix_tokens:].copy()


def positions_for(cfg: ModelConfig) -> tuple[np.ndarray, np.ndarray]:
    """(prefix_positions, chunk_positions): consecutive slots starting at 0."""
    p = np.arange(cfg.prefix_tokens + cfg.n_tokens, dtype=np.int32)
    return p[: cfg.prefix_tokens].copy(), p[cfg.prefix_tokens:].copy()


def gen_gemm_inputs(case: GemmCase, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """Activations x [m][k] (N(0,1) with 1% x20 outliers) and weights w [n][k] (N(0,0.02^2))."""
    gx = _gen(case.seed, f"gemm.x.{case.m}.{case.k}", device)
    x = torch.randn(case.m, case.k, generator=gx, device=device, dtype=torch.float32)
    u = torch.rand(case.m, case.k, generator=gx, device=device, dtype=torch.float32)
    x = torch.where(u < case.outlier_frac, x * case.outlier_scale, x)
    gw = _gen(case.seed, f"gemm.w.{case.n}.{case.k}", device)
    w = torch.randn(case.n, case.k, generator=gw, device=device, dtype=torch.float32)
    w.mul_(WEIGHT_STD)
    return x, w


def gen_normal(seed: int, name: str, shape, std: float = 1.0, device="cpu") -> torch.Tensor:
    """A generic seeded N(0, std^2) f32 tensor (used by the per-op test cases)."""
    g = _gen(seed, name, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t

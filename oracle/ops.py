"""The per-node operations of the Qwen2/Qwen3 prefill graph (oracle; test infrastructure).

Every node is evaluated in f64 from its f32 inputs and its output is rounded once
to f32, because the pages store every node output, the KV regions and the logits
as f32 (page "05 - Graph build - the IR and the builder": activations are [d, nt]
with token-major memory [nt][d], matmul outputs are DType::F32; page "09 - Prefill:
the first forward", section 2.5: K and V regions are n_kv_embd x n_ctx f32).

Pins live in tests/test_oracle_ops.py; each function's docstring names them.
"""
from __future__ import annotations

import math

import numpy as np

from .q8_0 import dequantize_q8_0, quantize_q8_0

f32, f64 = np.float32, np.float64


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma over the last axis.

    The "attn_norm" / "ffn_norm" / final-norm nodes of the layer listing (page
    "05 - Graph build", section 2.5; eps 1e-6 carried as an f32 payload, RmsNorm{eps}).
    Pinned by: unit RMS sqrt(ms / (ms + eps)) with gamma = 1, per-element gain.
    """
    x64 = np.asarray(x, dtype=f32).astype(f64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    y = x64 / np.sqrt(ms + f64(f32(eps))) * np.asarray(gamma, dtype=f32).astype(f64)
    return y.astype(f32)


def matmul_q8_0(x: np.ndarray, w_codes: np.ndarray, w_scales: np.ndarray,
                bias: np.ndarray | None = None) -> np.ndarray:
    """y[t, n] = sum_k dequant(Q8_0(x))[t, k] * dequant(W)[n, k] (+ b[n]).

    The matmul node quantizes its f32 input to Q8_0 on the fly (walkthrough index,
    stage 10) and multiplies by the quantized weight stored [out][in] (page "05 -
    Graph build", section 2.4 layout convention); the bias is applied inside the
    matmul (section 3.2, MatMulMeta.bias_name).  Each product of two dequantized
    values is exact in f64, so the f64 GEMM equals the per-block formula
    sum_kb d_x d_w sum q_x q_w up to f64 summation error.
    Pinned by: exact rational brute force on tiny shapes; single-block closed form.
    """
    xq, xd = quantize_q8_0(x)
    a = dequantize_q8_0(xq, xd)
    w = dequantize_q8_0(w_codes, w_scales)
    y = a @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=f32).astype(f64)
    return y.astype(f32)


def embed_q8_0(codes: np.ndarray, scales: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """h[t] = dequant(token_embd row ids[t]) (GetRows node 'embed', page "05", section 2.5)."""
    ids = np.asarray(ids, dtype=np.int64)
    return dequantize_q8_0(codes[ids], scales[ids]).astype(f32)


def qk_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over head_dim (Qwen3 QkNorm{hd, nh, eps}; page "05", sections 2.3, 2.6).

    x is [n, heads, hd]; gamma is [hd], shared by all heads.
    """
    return rms_norm(x, gamma, eps)


def rope_neox(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """NeoX rotary embedding of x [n, heads, hd] by the token positions.

    The rope nodes take the positions input as the rotation angle's source (page
    "09 - Prefill", section 2.2).  Style NeoX: within each head, pair i is
    (x_i, x_{i+hd/2}) for i < hd/2, rotated by angle pos * theta^(-2i/hd):
    (a, b) -> (a cos - b sin, a sin + b cos).
    Pinned by: identity at pos 0, pair norms kept, hand-worked pairing and
    frequency, scores depending only on the position difference.
    """
    n, heads, hd = x.shape
    half = hd // 2
    i = np.arange(half, dtype=f64)
    inv_freq = np.power(f64(f32(theta)), -2.0 * i / hd)
    ang = np.asarray(positions, dtype=f64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x64 = np.asarray(x, dtype=f32).astype(f64)
    a, b = x64[..., :half], x64[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1).astype(f32)


def kvcache_store(region_k: np.ndarray, region_v: np.ndarray, k: np.ndarray,
                  v: np.ndarray, positions: np.ndarray, n_ctx: int) -> None:
    """Row pos[t] of the layer's K (V) region <- rotated K[t] (raw V[t]), in place.

    Page "09 - Prefill", section 2.2: position p writes row p of the layer's K and V
    regions; section 3.4: a position >= n_ctx is a hard error, never a silent write.
    Page "05", section 3.2: the store reads the rotated K and the raw V.
    """
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size and (positions.min() < 0 or positions.max() >= n_ctx):
        raise ValueError(f"position out of range for n_ctx {n_ctx}")
    region_k[positions] = np.asarray(k, dtype=f32)
    region_v[positions] = np.asarray(v, dtype=f32)


def attention_gqa(q: np.ndarray, region_k: np.ndarray, region_v: np.ndarray,
                  positions: np.ndarray, n_head: int, n_head_kv: int, head_dim: int) -> np.ndarray:
    """Causal grouped-query attention over the layer's KV regions.

    o[t, h] = sum_{j <= pos[t]} softmax_j(q[t, h] . k_j / sqrt(hd)) v_j with the
    K/V head g = h // (n_head / n_head_kv): token t sees rows 0..=pos[t] (page "09 -
    Prefill", section 2.2, vl = pos[t] + 1), query heads share a KV head in
    contiguous groups (page "05", section 2.5: a group of 7 on the 0.5B), scale
    1/sqrt(hd).  Region rows are read after this call's stores (store before attention).
    Pinned by: V = 1 gives 1, one visible row gives v_0, uniform scores give the
    mean, head-to-group mapping, a loop-form brute force on a tiny case.
    """
    n = q.shape[0]
    group = n_head // n_head_kv
    positions = np.asarray(positions, dtype=np.int64)
    rows = int(positions.max()) + 1
    kk = region_k[:rows].astype(f64).reshape(rows, n_head_kv, head_dim)
    vv = region_v[:rows].astype(f64).reshape(rows, n_head_kv, head_dim)
    qq = np.asarray(q, dtype=f32).astype(f64).reshape(n, n_head, head_dim)
    visible = np.arange(rows)[None, :] <= positions[:, None]
    scale = 1.0 / math.sqrt(head_dim)
    out = np.empty((n, n_head, head_dim), dtype=f64)
    for h in range(n_head):
        g = h // group
        s = (qq[:, h, :] @ kk[:, g, :].T) * scale
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vv[:, g, :]
    return out.reshape(n, n_head * head_dim).astype(f32)


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up with silu(x) = x * sigmoid(x) (page "05", section 2.5, SwiGLU node)."""
    g = np.asarray(gate, dtype=f32).astype(f64)
    u = np.asarray(up, dtype=f32).astype(f64)
    with np.errstate(over="ignore"):
        s = g / (1.0 + np.exp(-g))
    return (s * u).astype(f32)


def add_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Residual add node: two f32 tensors, f32 result (one rounding)."""
    return (np.asarray(a, dtype=f32).astype(f64) + np.asarray(b, dtype=f32).astype(f64)).astype(f32)

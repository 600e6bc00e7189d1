"""The prefill forward of a Qwen2/Qwen3-style decoder, node by node (oracle).

Order of nodes per layer (page "05 - Graph build - the IR and the builder",
section 2.5 and the section 3.2 excerpts of the Qwen2 build):

    attn_norm -> Q, K, V matmuls (+bias) -> [Qwen3: per-head QK RMSNorm]
    -> rope(Q), rope(K) -> kvcache_store(rotated K, raw V, positions)
    -> attn(Q, region, positions) -> attn_output matmul -> h += .
    -> ffn_norm -> gate, up matmuls -> silu(gate) * up -> down matmul -> h += .

then output_norm and the lm_head matmul (token_embd when the embeddings are tied).

Tail rows (page "09 - Prefill: the first forward", section 2.4; page "05", section
2.8): in the last layer, right after the attention output projection, only the last
n_out rows of the projection and of the residual continue; the last FFN, the final
norm and lm_head run on those rows.  Every node after the cut is row-local, so the
result equals rows [nt - n_out, nt) of the full computation (pinned by a test).

Pre-flight (page "09", sections 3.2 and 3.4): every position must be < n_ctx and
n_out <= nt; the oracle raises before touching the regions.

The forward is pinned by its ops' pins, by token-by-token replay through the same
regions (page "09", section 2.3: the batched pass and the sequential one compute
the same thing), by future-token independence, by tail == full, and by a loop-form
brute force of a whole tiny model.  Its absolute logits on the synthetic models have
no external reference: parity of those values is pinned only through these checks.
"""
from __future__ import annotations

from typing import Mapping

import numpy as np

from . import ops
from .q8_0 import quantize_q8_0


class QuantizedWeights:
    """Name -> tensor view used by the forward.

    Matmul weights are returned as (codes int8 [out][in], scales f16 [out][in/32]);
    norm gains and biases as f32 arrays.  ``source`` maps a GGUF tensor name to its
    f32 values; weights are quantized with the oracle's own quantizer, lazily, and
    cached only when ``cache`` is true (large models re-quantize per access).
    """

    def __init__(self, source, q8_names, cache: bool = True):
        self._source = source
        self._q8 = set(q8_names)
        self._cache = {} if cache else None

    def __getitem__(self, name):
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        t = np.asarray(self._source(name), dtype=np.float32)
        val = quantize_q8_0(t) if name in self._q8 else t
        if self._cache is not None:
            self._cache[name] = val
        return val


def weights_from_arrays(arrays: Mapping[str, np.ndarray], q8_names) -> QuantizedWeights:
    return QuantizedWeights(lambda n: arrays[n], q8_names, cache=True)


def _mm(w, x, name, bias=None):
    codes, scales = w[name]
    return ops.matmul_q8_0(x, codes, scales, bias)


def prefill_forward(cfg, w, token_ids, positions, n_ctx: int, kv_k, kv_v,
                    n_out: int = 1, progress=None) -> np.ndarray:
    """Run one prefill call; returns logits f32 [n_out][vocab] and fills kv_k/kv_v.

    cfg: an object with n_layers, hidden, n_head, n_head_kv, head_dim, ffn, vocab,
    rms_eps, rope_theta, qkv_bias, qk_norm, tied.  kv_k / kv_v: per-layer f32 regions
    [n_ctx][n_head_kv * head_dim], updated in place (the caller owns them).
    progress: optional callable(layer_index) invoked after each layer (long runs report liveness).
    """
    ids = np.asarray(token_ids, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    nt = ids.shape[0]
    if nt < 1 or pos.shape[0] != nt:
        raise ValueError("need n_tokens >= 1 and one position per token")
    if not 1 <= n_out <= nt:
        raise ValueError("n_out must satisfy 1 <= n_out <= n_tokens")
    if pos.min() < 0 or pos.max() >= n_ctx:
        raise ValueError(f"position {pos.max()} exceeds n_ctx {n_ctx}")
    nh, nkv, hd, eps = cfg.n_head, cfg.n_head_kv, cfg.head_dim, cfg.rms_eps

    codes, scales = w["token_embd.weight"]
    h = ops.embed_q8_0(codes, scales, ids)
    for il in range(cfg.n_layers):
        p = f"blk.{il}."
        x = ops.rms_norm(h, w[p + "attn_norm.weight"], eps)
        bq = w[p + "attn_q.bias"] if cfg.qkv_bias else None
        bk = w[p + "attn_k.bias"] if cfg.qkv_bias else None
        bv = w[p + "attn_v.bias"] if cfg.qkv_bias else None
        q = _mm(w, x, p + "attn_q.weight", bq).reshape(nt, nh, hd)
        k = _mm(w, x, p + "attn_k.weight", bk).reshape(nt, nkv, hd)
        v = _mm(w, x, p + "attn_v.weight", bv)
        if cfg.qk_norm:
            q = ops.qk_norm(q, w[p + "attn_q_norm.weight"], eps)
            k = ops.qk_norm(k, w[p + "attn_k_norm.weight"], eps)
        q = ops.rope_neox(q, pos, cfg.rope_theta)
        k = ops.rope_neox(k, pos, cfg.rope_theta)
        ops.kvcache_store(kv_k[il], kv_v[il], k.reshape(nt, nkv * hd), v, pos, n_ctx)
        o = ops.attention_gqa(q.reshape(nt, nh * hd), kv_k[il], kv_v[il], pos, nh, nkv, hd)
        wo = _mm(w, o, p + "attn_output.weight")
        if il == cfg.n_layers - 1 and n_out < nt:
            wo, h = wo[nt - n_out:], h[nt - n_out:]   # tail rows (get_rows pair)
        h = ops.add_f32(h, wo)
        x = ops.rms_norm(h, w[p + "ffn_norm.weight"], eps)
        g = _mm(w, x, p + "ffn_gate.weight")
        u = _mm(w, x, p + "ffn_up.weight")
        s = ops.swiglu(g, u)
        h = ops.add_f32(h, _mm(w, s, p + "ffn_down.weight"))
        if progress is not None:
            progress(il)
    if cfg.n_layers == 0:
        h = h[nt - n_out:]
    x = ops.rms_norm(h, w["output_norm.weight"], eps)
    head = "token_embd.weight" if cfg.tied else "output.weight"
    return _mm(w, x, head)


def new_kv_regions(cfg, n_ctx: int, fill: float = 0.0):
    """Per-layer K and V regions, f32 [n_ctx][n_kv_embd], owned by the caller."""
    shape = (cfg.n_layers, n_ctx, cfg.n_head_kv * cfg.head_dim)
    return np.full(shape, fill, dtype=np.float32), np.full(shape, fill, dtype=np.float32)

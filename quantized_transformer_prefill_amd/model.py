"""A Qwen2/Qwen3-shaped model resident on one GPU, driven through the C ABI.

Loading quantizes every matmul weight with the library's own Q8_0 kernel (mi_quantize_q8_0)
and arranges the library layout: Q|K|V rows stacked, gate/up rows interleaved in groups of 32.
The model owns its workspace, RoPE table and KV regions; `forward` is one mi_prefill_forward.
"""
from __future__ import annotations

import ctypes as C
from typing import Callable, Iterable, Optional

import numpy as np
import torch

from . import binding as B


def interleave_gate_up(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """Rows 64p..64p+31 <- gate rows 32p.., rows 64p+32..64p+63 <- up rows 32p.. (any trailing dims)."""
    f = gate.shape[0]
    rest = gate.shape[1:]
    return torch.stack([gate.reshape(f // 32, 32, *rest), up.reshape(f // 32, 32, *rest)], dim=1).reshape(2 * f, *rest)


class PrefillModel:
    def __init__(self, cfg, tensors: Iterable, max_tokens: int, n_ctx: int, device="cuda",
                 kv_fill: float = 0.0):
        """cfg: shape/flags (synth.ModelConfig or alike); tensors: iterable of (name, kind, f32 tensor)."""
        self.cfg = cfg
        self.device = torch.device(device)
        self.max_tokens = max_tokens
        self.n_ctx = n_ctx
        q8, f32 = {}, {}
        for name, kind, t in tensors:
            t = t.to(self.device, torch.float32).contiguous()
            if kind == "q8":
                q8[name] = B.quantize_q8_0(t)
            else:
                f32[name] = t
            del t
        self.q8, self.f32 = q8, f32
        hp = B.Hparams(cfg.n_layers, cfg.hidden, cfg.n_head, cfg.n_head_kv, cfg.head_dim, cfg.ffn, cfg.vocab,
                       cfg.rms_eps, cfg.rope_theta, int(cfg.qkv_bias), int(cfg.qk_norm), int(cfg.tied))
        self.hp = hp
        keep = []
        self.layer_tensors = []
        layers = (B.LayerWeights * max(cfg.n_layers, 1))()
        for il in range(cfg.n_layers):
            p = f"blk.{il}."
            qc, qs = q8.pop(p + "attn_q.weight")
            kc, ks = q8.pop(p + "attn_k.weight")
            vc, vs = q8.pop(p + "attn_v.weight")
            wqkv = (torch.cat([qc, kc, vc]).contiguous(), torch.cat([qs, ks, vs]).contiguous())
            gc, gs = q8.pop(p + "ffn_gate.weight")
            uc, us = q8.pop(p + "ffn_up.weight")
            wgu = (interleave_gate_up(gc, uc).contiguous(), interleave_gate_up(gs, us).contiguous())
            wo = q8[p + "attn_output.weight"]
            wd = q8[p + "ffn_down.weight"]
            L = layers[il]
            L.wqkv, L.wo, L.w_gate_up, L.w_down = B.q8(*wqkv), B.q8(*wo), B.q8(*wgu), B.q8(*wd)
            if cfg.qkv_bias:
                bqkv = torch.cat([f32[p + "attn_q.bias"], f32[p + "attn_k.bias"], f32[p + "attn_v.bias"]]).contiguous()
                keep.append(bqkv)
                L.bqkv = bqkv.data_ptr()
            L.attn_norm = f32[p + "attn_norm.weight"].data_ptr()
            L.ffn_norm = f32[p + "ffn_norm.weight"].data_ptr()
            if cfg.qk_norm:
                L.q_norm = f32[p + "attn_q_norm.weight"].data_ptr()
                L.k_norm = f32[p + "attn_k_norm.weight"].data_ptr()
            keep += [wqkv, wgu]
            self.layer_tensors.append({"wqkv": wqkv, "w_gate_up": wgu, "wo": wo, "w_down": wd})
        self._keep, self._layers = keep, layers
        emb = q8["token_embd.weight"]
        out = emb if cfg.tied else q8["output.weight"]
        self.head = out
        rope_bytes = B.lib().mi_rope_table_bytes(C.byref(hp), n_ctx)
        self.rope = torch.empty(rope_bytes // 8, dtype=torch.float64, device=self.device)
        B.check(B.lib().mi_rope_table_init(C.byref(hp), n_ctx, self.rope.data_ptr(), B.stream_ptr()))
        ws_bytes = B.lib().mi_prefill_workspace_bytes(C.byref(hp), max_tokens)
        if ws_bytes == 0:
            B.check(B.MI_ERR_INVALID_ARG)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self.stage = B.Stage(hp, max_tokens)  # pinned host staging of ids and positions
        self.model = B.Model(hp, B.q8(*emb), B.q8(*out), f32["output_norm.weight"].data_ptr(),
                             C.cast(layers, C.POINTER(B.LayerWeights)), self.rope.data_ptr(), n_ctx,
                             self.workspace.data_ptr(), ws_bytes, max_tokens, None, self.stage.handle)
        kv_embd = cfg.n_head_kv * cfg.head_dim
        self.kv_k = torch.full((cfg.n_layers, n_ctx, kv_embd), kv_fill, dtype=torch.float32, device=self.device)
        self.kv_v = torch.full((cfg.n_layers, n_ctx, kv_embd), kv_fill, dtype=torch.float32, device=self.device)
        self._kv_ptrs_k = (C.c_void_p * max(cfg.n_layers, 1))(*[self.kv_k[i].data_ptr() for i in range(cfg.n_layers)])
        self._kv_ptrs_v = (C.c_void_p * max(cfg.n_layers, 1))(*[self.kv_v[i].data_ptr() for i in range(cfg.n_layers)])
        self.kv = B.KvRegions(self._kv_ptrs_k, self._kv_ptrs_v, cfg.n_layers, n_ctx, kv_embd)
        self.logits = torch.empty(cfg.vocab, dtype=torch.float32, device=self.device)

    def forward(self, token_ids, positions, n_ctx: Optional[int] = None, logits: Optional[torch.Tensor] = None):
        """One prefill call; returns device logits f32 [vocab] of the last token."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        out = self.logits if logits is None else logits
        self.model.stream = B.stream_ptr()
        B.check(B.lib().mi_prefill_forward(C.byref(self.model), ids.ctypes.data, pos.ctypes.data, ids.shape[0],
                                           self.n_ctx if n_ctx is None else n_ctx, C.byref(self.kv),
                                           out.data_ptr()))
        return out

    def new_kv_set(self, fill: float = 0.0) -> "KvSet":
        """Another sequence's KV regions (all layers, n_ctx rows), for forward_slots."""
        return KvSet(self.cfg, self.n_ctx, self.device, fill)

    def own_kv_set(self) -> "KvSet":
        """The model's own regions (kv_k / kv_v) as a KvSet."""
        ks = KvSet.__new__(KvSet)
        ks.k, ks.v, ks.regions, ks._pk, ks._pv = self.kv_k, self.kv_v, self.kv, self._kv_ptrs_k, self._kv_ptrs_v
        return ks

    def forward_slots(self, slots, n_ctx: Optional[int] = None) -> torch.Tensor:
        """Several sequences in one call (mi_prefill_forward_slots): `slots` is a list of
        (token_ids, positions, KvSet); returns device logits f32 [n_slots][vocab]."""
        ids = np.ascontiguousarray(np.concatenate([np.asarray(a, np.int32) for a, _, _ in slots]))
        pos = np.ascontiguousarray(np.concatenate([np.asarray(b, np.int32) for _, b, _ in slots]))
        counts = np.ascontiguousarray(np.array([len(a) for a, _, _ in slots], np.int32))
        kvs = (B.KvRegions * len(slots))(*[ks.regions for _, _, ks in slots])
        out = torch.empty(len(slots), self.cfg.vocab, dtype=torch.float32, device=self.device)
        self.model.stream = B.stream_ptr()
        B.check(B.lib().mi_prefill_forward_slots(C.byref(self.model), ids.ctypes.data, pos.ctypes.data,
                                                 counts.ctypes.data, len(slots),
                                                 self.n_ctx if n_ctx is None else n_ctx, kvs, out.data_ptr()))
        return out

    def decode(self, token_id: int, position: int, n_ctx: Optional[int] = None,
               logits: Optional[torch.Tensor] = None):
        """One decode step (mi_decode_step); returns device logits f32 [vocab]."""
        out = self.logits if logits is None else logits
        self.model.stream = B.stream_ptr()
        B.check(B.lib().mi_decode_step(C.byref(self.model), int(token_id), int(position),
                                       self.n_ctx if n_ctx is None else n_ctx, C.byref(self.kv), out.data_ptr()))
        return out

    def graph(self, n_tokens: int, n_out: int = 1) -> "PrefillGraph":
        """A captured forward for n_tokens-token calls on torch's current stream (see PrefillGraph)."""
        return PrefillGraph(self, n_tokens, n_out)

    def forward_n(self, token_ids, positions, n_out: int, n_ctx: Optional[int] = None):
        """One prefill call; returns device logits f32 [n_out][vocab] of the last n_out tokens."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        out = torch.empty(max(n_out, 1), self.cfg.vocab, dtype=torch.float32, device=self.device)
        self.model.stream = B.stream_ptr()
        B.check(B.lib().mi_prefill_forward_n(C.byref(self.model), ids.ctypes.data, pos.ctypes.data, ids.shape[0],
                                             self.n_ctx if n_ctx is None else n_ctx, C.byref(self.kv), n_out,
                                             out.data_ptr()))
        return out


class PrefillGraph:
    """mi_prefill_graph_* around a PrefillModel: the forward's kernels captured once, replayed per call.

    Capture happens on torch's current stream, which must not be the default stream; `launch` replays
    on that stream and returns the logits tensor (the same device buffer every call).
    """

    def __init__(self, model: PrefillModel, n_tokens: int, n_out: int = 1):
        self.model = model
        self.n_tokens, self.n_out = n_tokens, n_out
        self.logits = torch.empty(n_out, model.cfg.vocab, dtype=torch.float32, device=model.device)
        model.model.stream = B.stream_ptr()
        if not model.model.stream:
            raise ValueError("graph capture needs a non-default stream (use torch.cuda.stream(...))")
        h = C.c_void_p()
        B.check(B.lib().mi_prefill_graph_create(C.byref(model.model), n_tokens, model.n_ctx, C.byref(model.kv), n_out,
                                                self.logits.data_ptr(), C.byref(h)))
        self.handle = h

    def launch(self, token_ids, positions) -> torch.Tensor:
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        if ids.shape[0] != self.n_tokens or pos.shape[0] != self.n_tokens:
            raise ValueError(f"graph captured for {self.n_tokens} tokens")
        B.check(B.lib().mi_prefill_graph_launch(self.handle, ids.ctypes.data, pos.ctypes.data))
        return self.logits

    def nodes(self) -> int:
        """Kernel launches in the captured forward."""
        n = C.c_int32()
        B.check(B.lib().mi_prefill_graph_nodes(self.handle, C.byref(n)))
        return n.value

    def close(self):
        if self.handle:
            B.lib().mi_prefill_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KvSet:
    """One sequence's KV regions: f32 [n_layers][n_ctx][n_kv_embd] for K and V, plus the C descriptor."""

    def __init__(self, cfg, n_ctx: int, device, fill: float = 0.0):
        kv_embd = cfg.n_head_kv * cfg.head_dim
        self.k = torch.full((cfg.n_layers, n_ctx, kv_embd), fill, dtype=torch.float32, device=device)
        self.v = torch.full((cfg.n_layers, n_ctx, kv_embd), fill, dtype=torch.float32, device=device)
        self._pk = (C.c_void_p * max(cfg.n_layers, 1))(*[self.k[i].data_ptr() for i in range(cfg.n_layers)])
        self._pv = (C.c_void_p * max(cfg.n_layers, 1))(*[self.v[i].data_ptr() for i in range(cfg.n_layers)])
        self.regions = B.KvRegions(self._pk, self._pv, cfg.n_layers, n_ctx, kv_embd)

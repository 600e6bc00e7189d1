"""ctypes binding of libmi_prefill.so: argument marshalling only.

Every step of the forward runs in the library's HIP kernels; torch only provides device memory
and the current HIP stream.  Loading fails loudly when the built library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MI_PREFILL_LIB selects another build of the same library (for A/B timing of builds)
LIB_PATH = os.environ.get("MI_PREFILL_LIB") or os.path.join(_HERE, "libmi_prefill.so")

MI_OK, MI_ERR_INVALID_ARG, MI_ERR_POSITION_RANGE, MI_ERR_DUP_POSITION = 0, 1, 2, 3
MI_ERR_KV_MISMATCH, MI_ERR_WORKSPACE, MI_ERR_HIP, MI_ERR_UNSUPPORTED = 4, 5, 6, 7


class MiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mi_prefill error {code}: {msg}")
        self.code = code


class Hparams(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_head", C.c_int32),
                ("n_head_kv", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("qkv_bias", C.c_int32), ("qk_norm", C.c_int32), ("tied", C.c_int32)]


class Q8Matrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int32), ("cols", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [("wqkv", Q8Matrix), ("wo", Q8Matrix), ("w_gate_up", Q8Matrix), ("w_down", Q8Matrix),
                ("bqkv", C.c_void_p), ("attn_norm", C.c_void_p), ("ffn_norm", C.c_void_p),
                ("q_norm", C.c_void_p), ("k_norm", C.c_void_p)]


class Model(C.Structure):
    _fields_ = [("hp", Hparams), ("token_embd", Q8Matrix), ("output", Q8Matrix),
                ("output_norm", C.c_void_p), ("layers", C.POINTER(LayerWeights)),
                ("rope_table", C.c_void_p), ("rope_rows", C.c_int32), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("max_tokens", C.c_int32), ("stream", C.c_void_p),
                ("stage", C.c_void_p)]


class KvRegions(C.Structure):
    _fields_ = [("k", C.POINTER(C.c_void_p)), ("v", C.POINTER(C.c_void_p)), ("n_layers", C.c_int32),
                ("n_ctx", C.c_int32), ("n_kv_embd", C.c_int32)]


class SamplerParams(C.Structure):
    _fields_ = [("repeat_penalty", C.c_float), ("frequency_penalty", C.c_float), ("presence_penalty", C.c_float),
                ("top_k", C.c_int32), ("top_p", C.c_float), ("temperature", C.c_float)]


_P, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t

# name -> (restype, argtypes); mirrors include/mi_prefill.h
SIGNATURES = {
    "mi_prefill_workspace_bytes": (_SZ, [C.POINTER(Hparams), _I32]),
    "mi_stage_create": (C.c_int, [C.POINTER(Hparams), _I32, C.POINTER(C.c_void_p)]),
    "mi_stage_destroy": (None, [_P]),
    "mi_rope_table_bytes": (_SZ, [C.POINTER(Hparams), _I32]),
    "mi_rope_table_init": (C.c_int, [C.POINTER(Hparams), _I32, _P, _P]),
    "mi_prefill_forward": (C.c_int, [C.POINTER(Model), _P, _P, _I32, _I32, C.POINTER(KvRegions), _P]),
    "mi_prefill_forward_n": (C.c_int, [C.POINTER(Model), _P, _P, _I32, _I32, C.POINTER(KvRegions), _I32, _P]),
    "mi_decode_step": (C.c_int, [C.POINTER(Model), _I32, _I32, _I32, C.POINTER(KvRegions), _P]),
    "mi_prefill_forward_slots": (C.c_int, [C.POINTER(Model), _P, _P, _P, _I32, _I32, C.POINTER(KvRegions), _P]),
    "mi_prefill_graph_create": (C.c_int, [C.POINTER(Model), _I32, _I32, C.POINTER(KvRegions), _I32, _P,
                                          C.POINTER(C.c_void_p)]),
    "mi_prefill_graph_launch": (C.c_int, [_P, _P, _P]),
    "mi_prefill_graph_nodes": (C.c_int, [_P, C.POINTER(C.c_int32)]),
    "mi_prefill_graph_destroy": (None, [_P]),
    "mi_quantize_q8_0": (C.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "mi_pack_q8_0": (C.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "mi_gemm_q8_0": (C.c_int, [_P, _P, _I32, C.POINTER(Q8Matrix), _P, _P, _P, _P]),
    "mi_gemm_q8_0_ws": (C.c_int, [_P, _P, _I32, C.POINTER(Q8Matrix), _P, _P, _P, _P, _SZ, _I32, _P]),
    "mi_gemm_q8_0_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mi_gemm_q8_0_static": (C.c_int, [_P, _P, _I32, C.POINTER(Q8Matrix), _P, _P, _P, _I32, _P]),
    "mi_sampler_workspace_bytes": (_SZ, []),
    "mi_sample": (C.c_int, [_P, _I32, _P, _I32, C.POINTER(SamplerParams), C.c_uint64, C.c_uint64, _P, _SZ, _P, _P]),
    "mi_gemm_swiglu_q8_0": (C.c_int, [_P, _P, _I32, C.POINTER(Q8Matrix), _P, _P, _P, _SZ, _P]),
    "mi_rmsnorm_quant": (C.c_int, [_P, _P, _I64, _I32, _F, _P, _P, _P, _P]),
    "mi_qk_norm": (C.c_int, [_P, _P, _I64, _I32, _I32, _F, _P]),
    "mi_rope_kvstore": (C.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P, _I32, _P]),
    "mi_attention_gqa": (C.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "mi_swiglu_quant": (C.c_int, [_P, _P, _I64, _I32, _P, _P, _P]),
    "mi_embed_q8_0": (C.c_int, [C.POINTER(Q8Matrix), _P, _I32, _P, _P]),
    "mi_lm_head_row": (C.c_int, [_P, _P, _F, C.POINTER(Q8Matrix), _P, _P, _P]),
    "mi_last_error": (C.c_char_p, []),
    "mi_version": (C.c_char_p, []),
}

_lib = None


def lib() -> C.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m quantized_transformer_prefill_amd.build`")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(rc: int) -> None:
    if rc != MI_OK:
        raise MiError(rc, lib().mi_last_error().decode())


def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def stream_ptr() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype) -> None:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"expected a contiguous {dtype} device tensor, got {t.dtype} on {t.device}")


def q8(codes: torch.Tensor, scales: torch.Tensor) -> Q8Matrix:
    rows, cols = codes.shape
    return Q8Matrix(codes.data_ptr(), scales.data_ptr(), rows, cols)


# ---------------------------------------------------------------- per-op calls
def quantize_q8_0(x: torch.Tensor):
    _dev(x, torch.float32)
    rows, cols = x.reshape(-1, x.shape[-1]).shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device=x.device)
    check(lib().mi_quantize_q8_0(x.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), stream_ptr()))
    return codes, scales


def pack_q8_0(blocks: torch.Tensor, rows: int, cols: int):
    """Canonical 34-byte Q8_0 blocks (a device uint8 tensor of rows*cols/32*34 bytes) -> (codes, scales)."""
    _dev(blocks, torch.uint8)
    codes = torch.empty((rows, cols), dtype=torch.int8, device=blocks.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device=blocks.device)
    check(lib().mi_pack_q8_0(blocks.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), stream_ptr()))
    return codes, scales


class Stage:
    """mi_stage_create / mi_stage_destroy: the pinned host staging a model's forward calls go through."""

    def __init__(self, hp: Hparams, max_tokens: int):
        h = C.c_void_p()
        check(lib().mi_stage_create(C.byref(hp), max_tokens, C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            lib().mi_stage_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_q8_0(a_codes, a_scales, w_codes, w_scales, bias=None, residual=None, split_k: int = 1, out=None):
    m, n = a_codes.shape[0], w_codes.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a_codes.device)
    w = q8(w_codes, w_scales)
    if split_k == 1:
        check(lib().mi_gemm_q8_0(a_codes.data_ptr(), a_scales.data_ptr(), m, C.byref(w), ptr(bias), ptr(residual),
                                 out.data_ptr(), stream_ptr()))
    else:
        need = lib().mi_gemm_q8_0_workspace_bytes(m, n, a_codes.shape[1]) if split_k == 0 else \
            split_k * m * n * 8
        ws = torch.empty(max(need, 8), dtype=torch.uint8, device=a_codes.device)
        check(lib().mi_gemm_q8_0_ws(a_codes.data_ptr(), a_scales.data_ptr(), m, C.byref(w), ptr(bias), ptr(residual),
                                    out.data_ptr(), ws.data_ptr(), ws.numel(), split_k, stream_ptr()))
        out._mi_ws = ws  # keep alive until the stream has used it
    return out


def gemm_swiglu_q8_0(a_codes, a_scales, w_codes, w_scales, workspace=None):
    m, n2 = a_codes.shape[0], w_codes.shape[0]
    f = n2 // 2
    s_codes = torch.empty((m, f), dtype=torch.int8, device=a_codes.device)
    s_scales = torch.empty((m, f // 32), dtype=torch.int16, device=a_codes.device)
    w = q8(w_codes, w_scales)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    check(lib().mi_gemm_swiglu_q8_0(a_codes.data_ptr(), a_scales.data_ptr(), m, C.byref(w), s_codes.data_ptr(),
                                    s_scales.data_ptr(), ws_ptr, ws_bytes, stream_ptr()))
    return s_codes, s_scales


def rmsnorm_quant(x, gamma, eps, want_y=False):
    _dev(x, torch.float32)
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device=x.device)
    y = torch.empty_like(x) if want_y else None
    check(lib().mi_rmsnorm_quant(x.data_ptr(), gamma.data_ptr(), rows, cols, eps, codes.data_ptr(),
                                 scales.data_ptr(), ptr(y), stream_ptr()))
    return (codes, scales, y) if want_y else (codes, scales)


def qk_norm_(x, gamma, n_heads, head_dim, eps):
    _dev(x, torch.float32)
    check(lib().mi_qk_norm(x.data_ptr(), gamma.data_ptr(), x.shape[0], n_heads, head_dim, eps, stream_ptr()))
    return x


def rope_kvstore(q, k, v, positions_dev, n_head, n_head_kv, head_dim, table, table_rows, k_region, v_region):
    n = q.shape[0]
    check(lib().mi_rope_kvstore(q.data_ptr(), k.data_ptr(), v.data_ptr(), positions_dev.data_ptr(), n, n_head,
                                n_head_kv, head_dim, table.data_ptr(), table_rows, k_region.data_ptr(),
                                v_region.data_ptr(), k_region.shape[0], stream_ptr()))


def attention_gqa(q, k_region, v_region, positions_dev, max_pos, n_head, n_head_kv, head_dim):
    out = torch.empty_like(q)
    check(lib().mi_attention_gqa(q.data_ptr(), k_region.data_ptr(), v_region.data_ptr(), positions_dev.data_ptr(),
                                 q.shape[0], max_pos, n_head, n_head_kv, head_dim, k_region.shape[0],
                                 out.data_ptr(), stream_ptr()))
    return out


def swiglu_quant(gate, up):
    rows, cols = gate.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=gate.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device=gate.device)
    check(lib().mi_swiglu_quant(gate.data_ptr(), up.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                stream_ptr()))
    return codes, scales


def embed_q8_0(codes, scales, ids_dev):
    out = torch.empty((ids_dev.shape[0], codes.shape[1]), dtype=torch.float32, device=codes.device)
    t = q8(codes, scales)
    check(lib().mi_embed_q8_0(C.byref(t), ids_dev.data_ptr(), ids_dev.shape[0], out.data_ptr(), stream_ptr()))
    return out


def lm_head_row(x_row, gamma, eps, head_codes, head_scales):
    logits = torch.empty(head_codes.shape[0], dtype=torch.float32, device=x_row.device)
    scratch = torch.empty(head_codes.shape[1] * 2 + 512, dtype=torch.uint8, device=x_row.device)
    h = q8(head_codes, head_scales)
    check(lib().mi_lm_head_row(x_row.data_ptr(), gamma.data_ptr(), eps, C.byref(h), logits.data_ptr(),
                               scratch.data_ptr(), stream_ptr()))
    return logits


def sample(logits, window, params, seed: int, step: int, workspace=None, token_out=None) -> torch.Tensor:
    """mi_sample on device logits f32 [vocab]; `params` has the fields of SamplerParams; returns
    the device int32 [1] token."""
    _dev(logits, torch.float32)
    vocab = logits.numel()
    if workspace is None:
        workspace = torch.empty(lib().mi_sampler_workspace_bytes(), dtype=torch.uint8, device=logits.device)
    if token_out is None:
        token_out = torch.empty(1, dtype=torch.int32, device=logits.device)
    w = np.ascontiguousarray(np.asarray(window, dtype=np.int32).reshape(-1))
    sp = SamplerParams(params.repeat_penalty, params.frequency_penalty, params.presence_penalty, params.top_k,
                       params.top_p, params.temperature)
    check(lib().mi_sample(logits.data_ptr(), vocab, w.ctypes.data if w.size else None, w.size, C.byref(sp),
                          seed, step, workspace.data_ptr(), workspace.numel(), token_out.data_ptr(), stream_ptr()))
    return token_out

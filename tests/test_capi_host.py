"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and rejects
bad calls with the documented error codes before touching a device (no GPU needed)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from quantized_transformer_prefill_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_prefill.h")
PROBE_HEADER = os.path.join(ROOT, "include", "mi_probes.h")
PROBE_LIB = os.path.join(ROOT, "quantized_transformer_prefill_amd", "libmi_probes.so")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(mi_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 15, names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mi_prefill.h but not exported"
        assert n in B.SIGNATURES, f"{n} has no binding signature"
    assert lib.mi_version().startswith(b"mi_prefill")


def test_probe_library_exports_its_header():
    """libmi_probes.so (the rate probes behind the matmul's ceilings) loads and exports what
    mi_probes.h declares; bad arguments are refused before any launch."""
    names = declared_functions(PROBE_HEADER)
    assert names == ["mi_probe_run"], names
    lib = C.CDLL(PROBE_LIB)
    lib.mi_probe_run.restype = C.c_int
    lib.mi_probe_run.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.POINTER(C.c_double), C.c_void_p]
    w = C.c_double()
    assert lib.mi_probe_run(0, 0, 10, FAKE, C.byref(w), None) == B.MI_ERR_INVALID_ARG
    assert lib.mi_probe_run(0, 4, 10, None, C.byref(w), None) == B.MI_ERR_INVALID_ARG
    assert lib.mi_probe_run(99, 4, 10, FAKE, C.byref(w), None) == B.MI_ERR_INVALID_ARG


FAKE = 0x10000  # a non-null pointer value that is never dereferenced on these paths


def _fake_q8(rows, cols):
    return B.Q8Matrix(FAKE, FAKE, rows, cols)


def make_model(n_layers=2, hidden=64, nh=4, nkv=2, hd=64, ffn=96, vocab=50, max_tokens=8, n_ctx=16,
               ws_bytes=None):
    hp = B.Hparams(n_layers, hidden, nh, nkv, hd, ffn, vocab, 1e-6, 1e6, 1, 0, 0)
    layers = (B.LayerWeights * n_layers)()
    for L in layers:
        L.wqkv = _fake_q8(nh * hd + 2 * nkv * hd, hidden)
        L.wo = _fake_q8(hidden, nh * hd)
        L.w_gate_up = _fake_q8(2 * ffn, hidden)
        L.w_down = _fake_q8(hidden, ffn)
        L.bqkv = L.attn_norm = L.ffn_norm = FAKE
    need = B.lib().mi_prefill_workspace_bytes(C.byref(hp), max_tokens)
    model = B.Model(hp, _fake_q8(vocab, hidden), _fake_q8(vocab, hidden), FAKE,
                    C.cast(layers, C.POINTER(B.LayerWeights)), FAKE, n_ctx, FAKE,
                    need if ws_bytes is None else ws_bytes, max_tokens, None)
    region = 4 * n_ctx * nkv * hd  # distinct, non-overlapping fake regions (never dereferenced)
    kk = (C.c_void_p * n_layers)(*[FAKE + (2 * i) * region for i in range(n_layers)])
    vv = (C.c_void_p * n_layers)(*[FAKE + (2 * i + 1) * region for i in range(n_layers)])
    kv = B.KvRegions(kk, vv, n_layers, n_ctx, nkv * hd)
    return model, kv, (layers, kk, vv)


def call_forward(model, kv, ids, pos, n_ctx=16):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    return B.lib().mi_prefill_forward(C.byref(model), ids.ctypes.data, pos.ctypes.data, ids.shape[0], n_ctx,
                                      C.byref(kv), FAKE)


def test_forward_rejects_out_of_range_positions():
    model, kv, keep = make_model()
    assert call_forward(model, kv, [1, 2, 3], [0, 1, 16]) == B.MI_ERR_POSITION_RANGE
    assert b"position 16" in B.lib().mi_last_error()
    assert call_forward(model, kv, [1, 2, 3], [0, -1, 2]) == B.MI_ERR_POSITION_RANGE


def test_forward_rejects_duplicate_positions():
    model, kv, keep = make_model()
    assert call_forward(model, kv, [1, 2, 3], [4, 1, 4]) == B.MI_ERR_DUP_POSITION


def test_forward_rejects_kv_mismatch_and_sizes():
    model, kv, keep = make_model()
    assert call_forward(model, kv, [1, 2], [0, 1], n_ctx=15) == B.MI_ERR_KV_MISMATCH
    kv.n_kv_embd = 64
    assert call_forward(model, kv, [1, 2], [0, 1]) == B.MI_ERR_KV_MISMATCH
    model, kv, keep = make_model()
    assert call_forward(model, kv, list(range(9)), list(range(9))) == B.MI_ERR_WORKSPACE
    model, kv, keep = make_model(ws_bytes=100)
    assert call_forward(model, kv, [1], [0]) == B.MI_ERR_WORKSPACE
    model, kv, keep = make_model()
    assert call_forward(model, kv, [], []) == B.MI_ERR_INVALID_ARG
    assert call_forward(model, kv, [50], [0]) == B.MI_ERR_INVALID_ARG  # id outside vocab


def test_forward_rejects_bad_shapes():
    model, kv, keep = make_model()
    keep[0][1].w_down = _fake_q8(64, 64)  # ffn mismatch
    assert call_forward(model, kv, [1], [0]) == B.MI_ERR_INVALID_ARG
    hp = B.Hparams(1, 64, 4, 3, 64, 96, 50, 1e-6, 1e6, 0, 0, 0)  # 4 % 3 != 0
    assert B.lib().mi_prefill_workspace_bytes(C.byref(hp), 8) == 0
    hp = B.Hparams(1, 64, 4, 2, 96, 96, 50, 1e-6, 1e6, 0, 0, 0)  # head_dim 96 unsupported
    assert B.lib().mi_prefill_workspace_bytes(C.byref(hp), 8) == 0


def test_forward_n_and_graph_argument_checks():
    """n_out bounds and the graph entry points' host-side checks (nothing is captured or run)."""
    L = B.lib()
    model, kv, keep = make_model()
    ids = np.array([1, 2, 3], dtype=np.int32)
    pos = np.array([0, 1, 2], dtype=np.int32)
    for bad in (0, 4):
        assert L.mi_prefill_forward_n(C.byref(model), ids.ctypes.data, pos.ctypes.data, 3, 16, C.byref(kv), bad,
                                      FAKE) == B.MI_ERR_INVALID_ARG
    h = C.c_void_p(FAKE)
    assert L.mi_prefill_graph_create(C.byref(model), 3, 16, C.byref(kv), 1, FAKE, None) == B.MI_ERR_INVALID_ARG
    assert L.mi_prefill_graph_create(C.byref(model), 3, 15, C.byref(kv), 1, FAKE, C.byref(h)) == B.MI_ERR_KV_MISMATCH
    assert h.value is None  # the handle is cleared on error
    assert L.mi_prefill_graph_create(C.byref(model), 9, 16, C.byref(kv), 1, FAKE, C.byref(h)) == B.MI_ERR_WORKSPACE
    assert L.mi_prefill_graph_create(C.byref(model), 3, 16, C.byref(kv), 1, FAKE, C.byref(h)) == B.MI_ERR_INVALID_ARG
    assert b"non-default stream" in L.mi_last_error()
    assert L.mi_prefill_graph_launch(None, ids.ctypes.data, pos.ctypes.data) == B.MI_ERR_INVALID_ARG
    n = C.c_int32(-1)
    assert L.mi_prefill_graph_nodes(None, C.byref(n)) == B.MI_ERR_INVALID_ARG and n.value == -1
    L.mi_prefill_graph_destroy(None)  # a no-op


def test_per_op_argument_checks():
    L = B.lib()
    assert L.mi_quantize_q8_0(FAKE, 2, 48, FAKE, FAKE, None) == B.MI_ERR_INVALID_ARG
    w = _fake_q8(64, 48)
    assert L.mi_gemm_q8_0(FAKE, FAKE, 4, C.byref(w), None, None, FAKE, None) == B.MI_ERR_INVALID_ARG
    assert L.mi_attention_gqa(FAKE, FAKE, FAKE, FAKE, 3, 16, 4, 2, 64, 16, FAKE, None) == B.MI_ERR_POSITION_RANGE
    assert L.mi_rope_kvstore(FAKE, FAKE, FAKE, FAKE, 3, 4, 2, 64, FAKE, 8, FAKE, FAKE, 16, None) == \
        B.MI_ERR_INVALID_ARG  # rope table shorter than n_ctx
    gu = _fake_q8(96, 64)  # rows not a multiple of 64
    assert L.mi_gemm_swiglu_q8_0(FAKE, FAKE, 2, C.byref(gu), FAKE, FAKE, None, 0, None) == B.MI_ERR_INVALID_ARG


def test_workspace_grows_with_tokens():
    hp = B.Hparams(24, 896, 14, 2, 64, 4864, 151936, 1e-6, 1e6, 1, 0, 1)
    a = B.lib().mi_prefill_workspace_bytes(C.byref(hp), 16)
    b = B.lib().mi_prefill_workspace_bytes(C.byref(hp), 512)
    assert 0 < a < b
    assert B.lib().mi_rope_table_bytes(C.byref(hp), 4096) == 4096 * 32 * 2 * 8


def test_forward_rejects_rows_wider_than_the_one_row_kernels():
    """The one-row kernels of the last layer stage a whole Q8_0 input row in LDS: an attention
    output row (n_head * head_dim) or a SwiGLU row (ffn) above 49152 values is refused up front,
    before any layer is enqueued; 40 heads of 128 (5120 values) are accepted."""
    hp = B.Hparams(1, 4096, 40, 8, 128, 4096, 50, 1e-6, 1e6, 0, 1, 0)
    assert B.lib().mi_prefill_workspace_bytes(C.byref(hp), 8) > 0
    hp = B.Hparams(1, 4096, 32, 8, 128, 65536, 50, 1e-6, 1e6, 0, 1, 0)
    assert B.lib().mi_prefill_workspace_bytes(C.byref(hp), 8) == 0
    assert b"ffn" in B.lib().mi_last_error()
    hp = B.Hparams(1, 4096, 512, 8, 128, 4096, 50, 1e-6, 1e6, 0, 1, 0)
    assert B.lib().mi_prefill_workspace_bytes(C.byref(hp), 8) == 0
    model, kv, keep = make_model(hidden=4096, nh=32, nkv=8, hd=128, ffn=65536)
    assert call_forward(model, kv, [1], [0]) == B.MI_ERR_UNSUPPORTED


def test_forward_rejects_overlapping_regions():
    model, kv, keep = make_model()
    layers, kk, vv = keep
    vv[1] = kk[0]                       # V of layer 1 is K of layer 0
    assert call_forward(model, kv, [1, 2], [0, 1]) == B.MI_ERR_INVALID_ARG
    assert b"overlap" in B.lib().mi_last_error()
    model, kv, keep = make_model()
    layers, kk, vv = keep
    vv[0] = kk[0] + 4 * 64              # partly overlapping: shifted by one row
    assert call_forward(model, kv, [1, 2], [0, 1]) == B.MI_ERR_INVALID_ARG


def test_forward_needs_a_stage():
    model, kv, keep = make_model()
    assert call_forward(model, kv, [1, 2], [0, 1]) == B.MI_ERR_INVALID_ARG
    assert b"stage" in B.lib().mi_last_error()


def test_forward_rejects_shapes_past_32bit_offsets():
    """max_tokens x the widest activation row reaching 2^31 elements is refused on the host: the
    kernels address rows with 32-bit offsets."""
    hp = B.Hparams(2, 64, 4, 2, 64, 96, 50, 1e-6, 1e6, 1, 0, 0)
    max_tokens = (1 << 31) // 512 + 1   # the widest row here is Q|K|V: 4*64 + 2*2*64 = 512 values
    need = B.lib().mi_prefill_workspace_bytes(C.byref(hp), max_tokens)
    model, kv, keep = make_model(max_tokens=max_tokens, ws_bytes=need)
    assert call_forward(model, kv, [1, 2], [0, 1]) == B.MI_ERR_UNSUPPORTED
    assert b"2^31" in B.lib().mi_last_error()
    L = B.lib()
    w = _fake_q8(4096, 4096)
    assert L.mi_gemm_q8_0(FAKE, FAKE, 1 << 19, C.byref(w), None, None, FAKE, None) == B.MI_ERR_UNSUPPORTED
    assert L.mi_gemm_q8_0_ws(FAKE, FAKE, 1 << 19, C.byref(w), None, None, FAKE, None, 0, 0, None) == \
        B.MI_ERR_UNSUPPORTED
    gu = _fake_q8(1 << 17, 1 << 14)    # n * k = 2^31
    assert L.mi_gemm_swiglu_q8_0(FAKE, FAKE, 2, C.byref(gu), FAKE, FAKE, None, 0, None) == B.MI_ERR_UNSUPPORTED


def test_slots_reject_shared_regions():
    """Two sequences of one call must not share KV regions (their stores would race)."""
    model, kv, keep = make_model()
    ids = np.array([1, 2, 3], dtype=np.int32)
    pos = np.array([0, 1, 0], dtype=np.int32)
    counts = np.array([2, 1], dtype=np.int32)
    kvs = (B.KvRegions * 2)(kv, kv)     # the same region set twice
    rc = B.lib().mi_prefill_forward_slots(C.byref(model), ids.ctypes.data, pos.ctypes.data, counts.ctypes.data, 2,
                                          16, kvs, FAKE)
    assert rc == B.MI_ERR_INVALID_ARG and b"overlap" in B.lib().mi_last_error()


def test_pack_and_stage_argument_checks():
    L = B.lib()
    assert L.mi_pack_q8_0(FAKE, 4, 48, FAKE, FAKE, None) == B.MI_ERR_INVALID_ARG       # cols % 32
    assert L.mi_pack_q8_0(FAKE + 1, 4, 64, FAKE, FAKE, None) == B.MI_ERR_INVALID_ARG   # blocks odd address
    assert L.mi_pack_q8_0(FAKE, 4, 64, FAKE + 8, FAKE, None) == B.MI_ERR_INVALID_ARG   # codes not 16-aligned
    assert L.mi_pack_q8_0(FAKE, 0, 64, FAKE, FAKE, None) == B.MI_ERR_INVALID_ARG       # no rows
    hp = B.Hparams(2, 64, 4, 2, 64, 96, 50, 1e-6, 1e6, 1, 0, 0)
    assert L.mi_stage_create(C.byref(hp), 8, None) == B.MI_ERR_INVALID_ARG
    h = C.c_void_p(FAKE)
    assert L.mi_stage_create(C.byref(hp), 0, C.byref(h)) == B.MI_ERR_INVALID_ARG
    assert h.value is None
    bad = B.Hparams(2, 64, 4, 3, 64, 96, 50, 1e-6, 1e6, 1, 0, 0)
    assert L.mi_stage_create(C.byref(bad), 8, C.byref(h)) == B.MI_ERR_INVALID_ARG
    L.mi_stage_destroy(None)  # a no-op

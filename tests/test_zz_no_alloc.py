"""mi_gemm_q8_0_static -- the matmul that allocates nothing, its split-K partials in the library's
static device array -- against mi_gemm_q8_0_ws (the caller's workspace) on the same inputs and split,
through the C ABI: two calls in a row, the second on a smaller problem, bit for bit; the first also
against the oracle."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from oracle import ops
from oracle.q8_0 import quantize_q8_0
from quantized_transformer_prefill_amd import binding as B
from tests.gpu_util import assert_f32_match, need_gpu, say

pytestmark = pytest.mark.gpu


def _case(m, k, n, split, seed, dev, with_bias):
    x, _ = synth.gen_gemm_inputs(synth.GemmCase(m, k, 32, seed=seed), device=dev)
    w = synth.gen_normal(seed + 1, f"w{n}x{k}", (n, k), std=0.02, device=dev)
    bias = synth.gen_normal(seed + 2, f"b{n}", (n,), std=0.02, device=dev) if with_bias else None
    res = synth.gen_normal(seed + 3, f"r{m}x{n}", (m, n), device=dev)
    xc, xs = B.quantize_q8_0(x.contiguous())
    wc, wsc = B.quantize_q8_0(w)
    wm = B.q8(wc, wsc)
    L = B.lib()
    need = split * m * n * 8 if split > 1 else L.mi_gemm_q8_0_workspace_bytes(m, n, k)
    wsb = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    ref = torch.empty(m, n, dtype=torch.float32, device=dev)
    got = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    bp = None if bias is None else bias.data_ptr()
    B.check(L.mi_gemm_q8_0_ws(xc.data_ptr(), xs.data_ptr(), m, C.byref(wm), bp, res.data_ptr(), ref.data_ptr(),
                              wsb.data_ptr(), wsb.numel(), split, B.stream_ptr()))
    B.check(L.mi_gemm_q8_0_static(xc.data_ptr(), xs.data_ptr(), m, C.byref(wm), bp, res.data_ptr(), got.data_ptr(),
                                  split, B.stream_ptr()))
    torch.cuda.synchronize()
    return x, w, bias, res, ref.cpu().numpy(), got.cpu().numpy()


def test_static_scratch_matmul_equals_workspace_matmul():
    dev = need_gpu()
    # first: a long reduction over few rows, where the library splits K (f64 partials in the array)
    say("static-scratch gemm m=600 k=8192 n=1664 split=library")
    x, w, bias, res, ref, got = _case(600, 8192, 1664, 0, 41, dev, True)
    np.testing.assert_array_equal(got, ref)
    oq, od = quantize_q8_0(w.cpu().numpy())
    want = ops.add_f32(res.cpu().numpy(), ops.matmul_q8_0(x.cpu().numpy(), oq, od, bias.cpu().numpy()))
    assert_f32_match(got, want, what="static-scratch gemm vs oracle")
    # second, smaller, right after: an explicit split of 4 over the array the first call left behind
    say("static-scratch gemm m=100 k=2048 n=512 split=4")
    _, _, _, _, ref2, got2 = _case(100, 2048, 512, 4, 51, dev, False)
    np.testing.assert_array_equal(got2, ref2)
    assert np.all(np.isfinite(got2))


def test_static_scratch_rejects_oversized_split():
    dev = need_gpu()
    wc = torch.zeros(4096, 1024, dtype=torch.int8, device=dev)
    ws = torch.zeros(4096, 32, dtype=torch.int16, device=dev)
    wm = B.q8(wc, ws)
    out = torch.empty(2048, 4096, dtype=torch.float32, device=dev)
    a = torch.zeros(2048, 1024, dtype=torch.int8, device=dev)
    s = torch.zeros(2048, 32, dtype=torch.int16, device=dev)
    rc = B.lib().mi_gemm_q8_0_static(a.data_ptr(), s.data_ptr(), 2048, C.byref(wm), None, None, out.data_ptr(), 2,
                                     B.stream_ptr())
    assert rc == B.MI_ERR_WORKSPACE   # 2 x 2048 x 4096 f64 partials = 128 MiB > 64 MiB
    assert b"static scratch" in B.lib().mi_last_error()

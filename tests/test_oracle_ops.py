"""Pins of the oracle's per-node operations: closed forms, invariants, brute force."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import ops
from oracle.q8_0 import quantize_q8_0
from tests.exact import rn32

f32 = np.float32


# ---------------------------------------------------------------- Q8_0 matmul
def _exact_matmul(x, wq, wd, bias=None):
    """sum_kb d_x d_w sum q_x q_w (+b) on exact rationals, then RN to f32."""
    xq, xd = quantize_q8_0(x)
    m, k = x.shape
    n = wq.shape[0]
    out = np.zeros((m, n), dtype=np.float64)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kb in range(k // 32):
                dot = sum(int(xq[i, kb * 32 + t]) * int(wq[j, kb * 32 + t]) for t in range(32))
                acc += Fraction(float(xd[i, kb])) * Fraction(float(wd[j, kb])) * dot
            if bias is not None:
                acc += Fraction(float(bias[j]))
            out[i, j] = rn32(acc)
    return out


@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (3, 64, 5), (4, 96, 8)])
def test_matmul_matches_exact_rationals(m, k, n):
    rng = np.random.default_rng(m * 100 + n)
    x = rng.standard_normal((m, k)).astype(f32)
    x[0, 0] *= 20  # an outlier
    wq, wd = quantize_q8_0((rng.standard_normal((n, k)) * 0.02).astype(f32))
    bias = (rng.standard_normal(n) * 0.02).astype(f32)
    for b in (None, bias):
        got = ops.matmul_q8_0(x, wq, wd, b).astype(np.float64)
        want = _exact_matmul(x, wq, wd, b)
        ulp = np.spacing(np.abs(want).astype(f32)).astype(np.float64)
        assert np.all(np.abs(got - want) <= ulp), (got, want)


def test_matmul_single_block_closed_form():
    # one block: y = d_x * d_w * (integer dot); x chosen so that every code is known
    x = np.zeros((1, 32), dtype=f32)
    x[0, :4] = [127, 63.5, -1, 2]            # d_x = 1 -> codes 127, 64, -1, 2
    wq = np.zeros((1, 32), dtype=np.int8)
    wq[0, :4] = [1, -2, 3, 4]
    wd = np.array([[0.5]], dtype=np.float16)
    y = ops.matmul_q8_0(x, wq, wd)
    assert y[0, 0] == f32(1.0 * 0.5 * (127 - 128 - 3 + 8))


def test_matmul_is_dequant_matmul_within_f32_error():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 128)).astype(f32)
    wq, wd = quantize_q8_0((rng.standard_normal((10, 128)) * 0.02).astype(f32))
    xq, xd = quantize_q8_0(x)
    a = (xq.astype(f32).reshape(6, 4, 32) * xd.astype(f32)[..., None]).reshape(6, 128)
    w = (wq.astype(f32).reshape(10, 4, 32) * wd.astype(f32)[..., None]).reshape(10, 128)
    y32 = a @ w.T
    y = ops.matmul_q8_0(x, wq, wd)
    assert np.max(np.abs(y - y32)) <= 1e-5 * np.max(np.abs(y32))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_rms_closed_form():
    rng = np.random.default_rng(1)
    for scale in (1.0, 0.02, 1e-3):
        x = (rng.standard_normal((4, 896)) * scale).astype(f32)
        y = ops.rms_norm(x, np.ones(896, f32), 1e-6).astype(np.float64)
        ms = np.mean(x.astype(np.float64) ** 2, axis=1)
        want = np.sqrt(ms / (ms + float(f32(1e-6))))
        got = np.sqrt(np.mean(y ** 2, axis=1))
        np.testing.assert_allclose(got, want, rtol=1e-6)


def test_rmsnorm_gain_is_elementwise():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 64)).astype(f32)
    g = (1 + 0.5 * rng.standard_normal(64)).astype(f32)
    y1 = ops.rms_norm(x, np.ones(64, f32), 1e-6).astype(np.float64)
    y2 = ops.rms_norm(x, g, 1e-6).astype(np.float64)
    np.testing.assert_allclose(y2, y1 * g, rtol=2e-7)


def test_rmsnorm_hand_example():
    x = np.array([[3.0, 4.0]], dtype=f32)          # mean square 12.5
    y = ops.rms_norm(x, np.array([1.0, 2.0], f32), 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_array_equal(y, np.array([[f32(3 / r), f32(8 / r)]]))


# ---------------------------------------------------------------- RoPE (NeoX)
def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 4, 64)).astype(f32)
    np.testing.assert_array_equal(ops.rope_neox(x, np.array([0]), 1e6), x)


def test_rope_pairs_and_frequency_by_hand():
    # hd = 4: pairs (0, 2) and (1, 3); angles pos * theta^0 and pos * theta^-1/2
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]], dtype=f32)
    y = ops.rope_neox(x, np.array([1]), 1e6)
    np.testing.assert_array_equal(y[0, 0], np.array([math.cos(1), 0, math.sin(1), 0], dtype=f32))
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]], dtype=f32)
    y = ops.rope_neox(x, np.array([1000]), 1e6)      # 1000 * 1e6^-0.5 = 1 rad
    np.testing.assert_allclose(y[0, 0], [0, math.cos(1), 0, math.sin(1)], atol=1e-7)


def test_rope_keeps_pair_norms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 2, 128)).astype(f32)
    pos = np.array([0, 1, 17, 999, 4095])
    y = ops.rope_neox(x, pos, 1e6).astype(np.float64)
    x64 = x.astype(np.float64)
    n_in = x64[..., :64] ** 2 + x64[..., 64:] ** 2
    n_out = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-6)


def test_rope_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 64)).astype(f32)
    k = rng.standard_normal((1, 1, 64)).astype(f32)
    dots = []
    for a, b in [(10, 3), (107, 100), (4007, 4000)]:
        qa = ops.rope_neox(q, np.array([a]), 1e6).astype(np.float64)
        kb = ops.rope_neox(k, np.array([b]), 1e6).astype(np.float64)
        dots.append(float(np.sum(qa * kb)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-5)


# ---------------------------------------------------------------- attention
def _attn_loops(q, kreg, vreg, pos, nh, nkv, hd):
    out = np.zeros((len(pos), nh * hd))
    for t, p in enumerate(pos):
        for h in range(nh):
            g = h // (nh // nkv)
            s = [sum(float(q[t, h * hd + i]) * float(kreg[j, g * hd + i]) for i in range(hd)) / math.sqrt(hd)
                 for j in range(p + 1)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            for i in range(hd):
                out[t, h * hd + i] = sum(e[j] / z * float(vreg[j, g * hd + i]) for j in range(p + 1))
    return out.astype(f32)


def test_attention_matches_loop_form():
    rng = np.random.default_rng(8)
    nh, nkv, hd, n_ctx = 4, 2, 8, 12
    pos = np.array([2, 5, 6, 9])
    q = rng.standard_normal((4, nh * hd)).astype(f32)
    kreg = rng.standard_normal((n_ctx, nkv * hd)).astype(f32)
    vreg = rng.standard_normal((n_ctx, nkv * hd)).astype(f32)
    got = ops.attention_gqa(q, kreg, vreg, pos, nh, nkv, hd)
    want = _attn_loops(q, kreg, vreg, pos, nh, nkv, hd)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


def test_attention_constant_values_and_single_row():
    rng = np.random.default_rng(9)
    nh, nkv, hd = 6, 2, 16
    q = rng.standard_normal((3, nh * hd)).astype(f32)
    kreg = rng.standard_normal((8, nkv * hd)).astype(f32)
    ones = np.ones((8, nkv * hd), f32)
    out = ops.attention_gqa(q, kreg, ones, np.array([0, 3, 7]), nh, nkv, hd)
    np.testing.assert_allclose(out, 1.0, rtol=1e-7)          # softmax rows sum to 1
    vreg = rng.standard_normal((8, nkv * hd)).astype(f32)
    out = ops.attention_gqa(q[:1], kreg, vreg, np.array([0]), nh, nkv, hd)
    for h in range(nh):                                        # one visible row -> v_0
        g = h // 3
        np.testing.assert_array_equal(out[0, h * hd:(h + 1) * hd], vreg[0, g * hd:(g + 1) * hd])


def test_attention_uniform_scores_give_mean_and_group_mapping():
    nh, nkv, hd = 14, 2, 4                                     # groups of 7, as on the 0.5B
    q = np.zeros((1, nh * hd), f32)                           # all scores 0
    kreg = np.ones((5, nkv * hd), f32)
    vreg = np.zeros((5, nkv * hd), f32)
    vreg[:, :hd] = np.arange(5, dtype=f32)[:, None]           # group 0: rows 0..4
    vreg[:, hd:] = 10 * np.arange(5, dtype=f32)[:, None]      # group 1
    out = ops.attention_gqa(q, kreg, vreg, np.array([3]), nh, nkv, hd).reshape(nh, hd)
    np.testing.assert_allclose(out[:7], 1.5, rtol=1e-7)      # mean of 0..3
    np.testing.assert_allclose(out[7:], 15.0, rtol=1e-7)


def test_attention_ignores_rows_after_position():
    rng = np.random.default_rng(10)
    nh, nkv, hd = 2, 1, 8
    q = rng.standard_normal((2, nh * hd)).astype(f32)
    kreg = rng.standard_normal((6, nkv * hd)).astype(f32)
    vreg = rng.standard_normal((6, nkv * hd)).astype(f32)
    a = ops.attention_gqa(q, kreg, vreg, np.array([1, 5]), nh, nkv, hd)
    kreg2, vreg2 = kreg.copy(), vreg.copy()
    kreg2[2:] = 99.0
    vreg2[2:] = -7.0
    b = ops.attention_gqa(q[:1], kreg2, vreg2, np.array([1]), nh, nkv, hd)
    np.testing.assert_array_equal(a[0], b[0])


# ---------------------------------------------------------------- KV store, SwiGLU, embed
def test_kv_store_rows_and_range_check():
    kr = np.zeros((8, 4), f32)
    vr = np.zeros((8, 4), f32)
    k = np.arange(12, dtype=f32).reshape(3, 4)
    v = -k
    ops.kvcache_store(kr, vr, k, v, np.array([5, 0, 7]), 8)
    np.testing.assert_array_equal(kr[[5, 0, 7]], k)
    np.testing.assert_array_equal(vr[[5, 0, 7]], v)
    assert np.all(kr[[1, 2, 3, 4, 6]] == 0)
    with pytest.raises(ValueError):
        ops.kvcache_store(kr, vr, k, v, np.array([5, 0, 8]), 8)


def test_swiglu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 30.0, -60.0], f32)
    u = np.array([5.0, 2.0, 2.0, 0.5, 3.0], f32)
    s = ops.swiglu(g, u)
    sig = lambda x: 1 / (1 + math.exp(-x))
    want = [0.0, 2 * sig(1), -2 * sig(-1), 0.5 * 30 * sig(30), 3 * -60 * sig(-60)]
    np.testing.assert_allclose(s, np.array(want, f32), rtol=1e-7, atol=1e-30)


def test_embedding_dequantizes_rows():
    rng = np.random.default_rng(12)
    wq, wd = quantize_q8_0((rng.standard_normal((7, 64)) * 0.02).astype(f32))
    ids = np.array([6, 0, 6, 3])
    h = ops.embed_q8_0(wq, wd, ids)
    for t, i in enumerate(ids):
        for c in range(64):
            assert h[t, c] == f32(float(wd[i, c // 32]) * int(wq[i, c]))

"""Pins of the oracle's whole prefill forward: invariants the pages state, a loop-form
brute force of a tiny model, and the sizes the pages print."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.exact import q8_0_block_exact

f32 = np.float32

TINY = synth.ModelConfig(name="tiny", n_layers=2, hidden=64, n_head=4, n_head_kv=2, head_dim=16,
                         ffn=96, vocab=50, n_tokens=7, n_ctx=16, seed=5, qkv_bias=True)
TINY_Q3 = TINY.with_(name="tiny_qk", qkv_bias=False, qk_norm=True, tied=True, seed=6)


def build(cfg):
    arrays = {n: t.numpy() for n, k, t in synth.iter_tensors(cfg)}
    q8 = [n for n, s, k in synth.tensor_specs(cfg) if k == "q8"]
    return arrays, oracle.weights_from_arrays(arrays, q8)


def run(cfg, w, ids, pos, kv=None, n_out=1):
    if kv is None:
        kv = oracle.new_kv_regions(cfg, cfg.n_ctx)
    logits = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kv[0], kv[1], n_out=n_out)
    return logits, kv


@pytest.mark.parametrize("cfg", [TINY, TINY_Q3], ids=lambda c: c.name)
def test_prefill_equals_token_by_token_replay(cfg):
    _, w = build(cfg)
    ids = np.array([3, 17, 41, 0, 8, 49, 22])
    pos = np.arange(7)
    full, kv_a = run(cfg, w, ids, pos)
    kv_b = oracle.new_kv_regions(cfg, cfg.n_ctx)
    for t in range(7):
        step, _ = run(cfg, w, ids[t:t + 1], pos[t:t + 1], kv_b)
    np.testing.assert_allclose(step, full, rtol=0, atol=1e-6)
    np.testing.assert_allclose(kv_b[0], kv_a[0], rtol=0, atol=1e-6)
    np.testing.assert_allclose(kv_b[1], kv_a[1], rtol=0, atol=1e-6)


def test_chunked_prefill_equals_one_shot():
    cfg = TINY
    _, w = build(cfg)
    ids = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
    pos = np.arange(10)
    one, kv1 = run(cfg, w, ids, pos)
    kv2 = oracle.new_kv_regions(cfg, cfg.n_ctx)
    run(cfg, w, ids[:4], pos[:4], kv2)
    two, _ = run(cfg, w, ids[4:], pos[4:], kv2)
    np.testing.assert_allclose(two, one, rtol=0, atol=1e-6)
    np.testing.assert_allclose(kv2[0], kv1[0], rtol=0, atol=1e-6)


def test_tail_rows_equal_full_rows():
    _, w = build(TINY)
    ids = np.array([5, 4, 3, 2, 1, 0, 9])
    full, _ = run(TINY, w, ids, np.arange(7), n_out=7)
    for n_out in (1, 3):
        tail, _ = run(TINY, w, ids, np.arange(7), n_out=n_out)
        np.testing.assert_array_equal(tail, full[7 - n_out:])


def test_future_tokens_do_not_change_earlier_rows():
    _, w = build(TINY)
    ids = np.array([5, 4, 3, 2, 1, 0, 9])
    _, kv_a = run(TINY, w, ids, np.arange(7))
    ids2 = ids.copy()
    ids2[5:] = [33, 44]
    _, kv_b = run(TINY, w, ids2, np.arange(7))
    for layer in range(TINY.n_layers):
        np.testing.assert_array_equal(kv_a[0][layer, :5], kv_b[0][layer, :5])
        np.testing.assert_array_equal(kv_a[1][layer, :5], kv_b[1][layer, :5])
        assert not np.array_equal(kv_a[0][layer, 5:7], kv_b[0][layer, 5:7])


def test_positions_beyond_context_are_rejected_before_any_write():
    _, w = build(TINY)
    kv = oracle.new_kv_regions(TINY, TINY.n_ctx, fill=7.0)
    with pytest.raises(ValueError):
        run(TINY, w, np.array([1, 2]), np.array([3, TINY.n_ctx]), kv)
    assert np.all(kv[0] == 7.0) and np.all(kv[1] == 7.0)
    with pytest.raises(ValueError):
        run(TINY, w, np.array([1, 2]), np.array([0, 1]), kv, n_out=3)


# ---------------------------------------------------------------- loop-form brute force
def _q8_rows(mat):
    """Q8_0 of each row with the exact-rational quantizer; returns dequantized f64 rows."""
    out = []
    for row in mat:
        vals = []
        for b in range(0, len(row), 32):
            codes, d16 = q8_0_block_exact(row[b:b + 32])
            vals += [d16 * c for c in codes]
        out.append(vals)
    return out


def _loop_forward(cfg, arrays, ids, pos):
    """The whole forward with python loops and math; weights re-quantized independently."""
    hd, nh, nkv, eps = cfg.head_dim, cfg.n_head, cfg.n_head_kv, float(f32(cfg.rms_eps))
    W = {n: _q8_rows(arrays[n].tolist()) for n, s, k in synth.tensor_specs(cfg) if k == "q8"}
    r32 = lambda v: float(f32(v))

    def norm(x, g):
        ms = sum(v * v for v in x) / len(x)
        return [r32(x[i] / math.sqrt(ms + eps) * float(g[i])) for i in range(len(x))]

    def mm(x, name, bias=None):
        xq = _q8_rows([x])[0]
        return [r32(sum(a * b for a, b in zip(xq, wrow)) + (float(bias[j]) if bias is not None else 0.0))
                for j, wrow in enumerate(W[name])]

    def rope(x, p):
        out = list(x)
        for h in range(len(x) // hd):
            for i in range(hd // 2):
                a, b = x[h * hd + i], x[h * hd + i + hd // 2]
                ang = p * cfg.rope_theta ** (-2 * i / hd)
                out[h * hd + i] = r32(a * math.cos(ang) - b * math.sin(ang))
                out[h * hd + i + hd // 2] = r32(a * math.sin(ang) + b * math.cos(ang))
        return out

    kreg = [[None] * cfg.n_ctx for _ in range(cfg.n_layers)]
    vreg = [[None] * cfg.n_ctx for _ in range(cfg.n_layers)]
    H = [[d for d in W["token_embd.weight"][i]] for i in ids]
    for l in range(cfg.n_layers):
        p = f"blk.{l}."
        Q = []
        for t in range(len(ids)):
            x = norm(H[t], arrays[p + "attn_norm.weight"])
            b = (lambda n: arrays[p + n]) if cfg.qkv_bias else (lambda n: None)
            q = mm(x, p + "attn_q.weight", b("attn_q.bias"))
            k = mm(x, p + "attn_k.weight", b("attn_k.bias"))
            v = mm(x, p + "attn_v.weight", b("attn_v.bias"))
            if cfg.qk_norm:
                q = sum((norm(q[h * hd:(h + 1) * hd], arrays[p + "attn_q_norm.weight"]) for h in range(nh)), [])
                k = sum((norm(k[h * hd:(h + 1) * hd], arrays[p + "attn_k_norm.weight"]) for h in range(nkv)), [])
            Q.append(rope(q, pos[t]))
            kreg[l][pos[t]] = rope(k, pos[t])
            vreg[l][pos[t]] = v
        for t in range(len(ids)):
            o = []
            for h in range(nh):
                g = h // (nh // nkv)
                s = [sum(Q[t][h * hd + i] * kreg[l][j][g * hd + i] for i in range(hd)) / math.sqrt(hd)
                     for j in range(pos[t] + 1)]
                mx = max(s)
                e = [math.exp(v - mx) for v in s]
                z = sum(e)
                o += [r32(sum(e[j] / z * vreg[l][j][g * hd + i] for j in range(pos[t] + 1))) for i in range(hd)]
            wo = mm(o, p + "attn_output.weight")
            H[t] = [r32(a + b) for a, b in zip(H[t], wo)]
            x = norm(H[t], arrays[p + "ffn_norm.weight"])
            gate, up = mm(x, p + "ffn_gate.weight"), mm(x, p + "ffn_up.weight")
            s = [r32(gv / (1 + math.exp(-gv)) * uv) for gv, uv in zip(gate, up)]
            H[t] = [r32(a + b) for a, b in zip(H[t], mm(s, p + "ffn_down.weight"))]
    x = norm(H[-1], arrays["output_norm.weight"])
    return np.array(mm(x, "token_embd.weight" if cfg.tied else "output.weight"), dtype=f32)


@pytest.mark.parametrize("cfg", [TINY.with_(hidden=32, ffn=64, n_head=2, n_head_kv=1, vocab=11, n_layers=1),
                                 TINY_Q3.with_(hidden=32, ffn=64, n_head=2, n_head_kv=1, vocab=11, n_layers=2)],
                         ids=["qwen2_like", "qwen3_like"])
def test_forward_matches_loop_form_brute_force(cfg):
    arrays, w = build(cfg)
    ids = np.array([3, 10, 0])
    pos = np.array([0, 1, 2])
    got, _ = run(cfg, w, ids, pos)
    want = _loop_forward(cfg, arrays, ids, pos)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-6)


# ---------------------------------------------------------------- sizes printed on the pages
def test_sizes_printed_on_the_pages():
    # "09 - Prefill", section 2.5: 0.5B KV = 24 KB per token, ~96 MB at n_ctx 4096;
    # Qwen3-4B (36 layers x 1024-wide KV, the same KV shape as the 8B config) = 288 KB/token.
    assert synth.QWEN2_0P5B.kv_bytes_per_token() == 24 * 1024
    assert synth.QWEN2_0P5B.kv_bytes_per_token() * 4096 == 96 * 1024 * 1024
    assert synth.QWEN3_8B.kv_bytes_per_token() == 288 * 1024
    # section 2.6: one row of logits is 151,936 x 4 = 607,744 bytes
    assert synth.QWEN2_0P5B.vocab * 4 == 607744
    # section 2.4 / page "05" section 2.8: lm_head work, 30-token prompt vs last row only
    assert abs(30 * 896 * 151936 - 4.1e9) < 0.05e9
    assert abs(896 * 151936 - 1.4e8) < 0.05e8
    # page "05" section 3.1: one layer's K region is [128, 4096] f32 = 2 MB
    assert synth.QWEN2_0P5B.n_kv_embd * 4096 * 4 == 2 * 1024 * 1024

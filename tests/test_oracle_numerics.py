"""Why every node of the GPU path is computed to f64 accuracy and rounded once to f32.

Every matmul input is re-quantized to Q8_0, so an f32 value that moves by one unit in the last
place can flip a code that sits near a rounding tie; the flipped code moves its activation by a
whole quantization step, which moves the next layer's inputs and flips more codes.  Noise at the
level of f32 rounding (what two f32 summation orders differ by) therefore grows through the layers
past the logits bar (rel-L2 1e-3), while noise at the f64 level leaves the f32 node outputs, and so
everything downstream, unchanged.  These tests plant that noise in the oracle (on the CPU): every
matmul and attention output is multiplied by (1 + eps * N(0, 1)) before its f32 rounding."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import ops

MODEL = synth.ModelConfig(name="noise_probe", n_layers=4, hidden=896, n_head=14, n_head_kv=2, head_dim=64,
                          ffn=4864, vocab=8192, n_tokens=128, n_ctx=128, seed=5, qkv_bias=True, tied=False)


@pytest.fixture(scope="module")
def weights():
    host = {name: t.numpy() for name, kind, t in synth.iter_tensors(MODEL, device="cpu")}
    q8 = [n for n, s, k in synth.tensor_specs(MODEL) if k == "q8"]
    return oracle.weights_from_arrays(host, q8)


def logits_with_noise(monkeypatch, w, n_layers, eps):
    cfg = MODEL.with_(n_layers=n_layers)
    rng = np.random.default_rng(123)
    mm, att = ops.matmul_q8_0, ops.attention_gqa

    def jitter(y):
        if eps == 0.0:
            return y
        y64 = np.asarray(y, np.float32).astype(np.float64)
        return (y64 * (1.0 + eps * rng.standard_normal(y64.shape))).astype(np.float32)

    monkeypatch.setattr(ops, "matmul_q8_0", lambda *a, **k: jitter(mm(*a, **k)))
    monkeypatch.setattr(ops, "attention_gqa", lambda *a, **k: jitter(att(*a, **k)))
    try:
        _, ids = synth.gen_token_ids(cfg)
        _, pos = synth.positions_for(cfg)
        kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx)
        return oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0].astype(np.float64)
    finally:
        monkeypatch.setattr(ops, "matmul_q8_0", mm)
        monkeypatch.setattr(ops, "attention_gqa", att)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_f32_level_noise_breaks_the_logits_bar(weights, monkeypatch):
    clean = logits_with_noise(monkeypatch, weights, 4, 0.0)
    noisy = logits_with_noise(monkeypatch, weights, 4, 1e-7)
    r = rel_l2(noisy, clean)
    print(f"4 layers x 896, 1e-7 relative noise: logits rel-L2 {r:.3e}, max-abs {np.abs(noisy - clean).max():.3e}")
    assert r > 1e-3


def test_noise_grows_with_depth(weights, monkeypatch):
    """One layer: the 1e-7 noise reaches the logits at about its own size (few codes flip in one
    layer's inputs, and no later layer amplifies them)."""
    clean = logits_with_noise(monkeypatch, weights, 1, 0.0)
    noisy = logits_with_noise(monkeypatch, weights, 1, 1e-7)
    r = rel_l2(noisy, clean)
    print(f"1 layer, 1e-7 relative noise: logits rel-L2 {r:.3e}")
    assert r < 1e-4


def test_f64_level_noise_changes_nothing(weights, monkeypatch):
    clean = logits_with_noise(monkeypatch, weights, 4, 0.0)
    noisy = logits_with_noise(monkeypatch, weights, 4, 1e-15)
    r = rel_l2(noisy, clean)
    print(f"4 layers x 896, 1e-15 relative noise: logits rel-L2 {r:.3e}")
    assert r < 1e-6

"""Decode step (mi_decode_step: one token at one position) against the oracle's forward of the
same token at the same position over the same KV regions, after a prefill of the prompt."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_transformer_prefill_amd import binding as B
from tests.gpu_util import assert_f32_match, need_gpu, say
from tests.test_forward_gpu import SENTINEL, TINY_Q2, TINY_Q3, _random_tiny_configs, compare_logits, load_pair

pytestmark = pytest.mark.gpu


def decode_tokens(cfg, n_steps):
    """Token ids for the steps after the prompt (seeded, uniform like the prompt)."""
    rng = np.random.default_rng(cfg.seed + 1000)
    return rng.integers(0, cfg.vocab, size=n_steps).astype(np.int32)


def prefill_then_decode(cfg, dev, n_steps, graph=False):
    """Prefill the prompt on both sides, then n_steps decode steps at the following positions.
    Returns per-step (gpu logits, oracle logits) and the final regions of both sides."""
    m, w = load_pair(cfg, dev, max_tokens=cfg.prefix_tokens + cfg.n_tokens)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    if cfg.prefix_tokens:
        m.forward(pre_ids, pre_pos)
        oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
    m.forward(ids, pos)
    oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)
    p0 = int(pos[-1]) + 1
    toks = decode_tokens(cfg, n_steps)
    steps = []
    g = None
    if graph:
        torch.cuda.synchronize()  # the prefill above ran on the default stream
        stream = torch.cuda.Stream()
        torch.cuda.set_stream(stream)
        g = m.graph(1)
    try:
        for i, tok in enumerate(toks):
            p = p0 + i
            say(f"decode {cfg.name} step {i} token {int(tok)} position {p}")
            if graph:
                got = g.launch([tok], [p]).cpu().numpy().copy()
                _ = torch.ones(1000, device=dev).sum().item()   # unrelated eager work between replays
            else:
                got = m.decode(int(tok), p).cpu().numpy().copy()
            want = oracle.prefill_forward(cfg, w, np.array([tok], np.int32), np.array([p], np.int32), cfg.n_ctx,
                                          kk, vv)[0]
            steps.append((got, want))
    finally:
        if g is not None:
            g.close()
            torch.cuda.set_stream(torch.cuda.default_stream())
    torch.cuda.synchronize()
    return m, steps, kk, vv, p0 + n_steps


# 40 query heads of 128: an attention output row of 5120 values, wider than the hidden size
TINY_WIDE = synth.ModelConfig(name="tiny_wide_heads", n_layers=2, hidden=256, n_head=40, n_head_kv=8, head_dim=128,
                              ffn=384, vocab=1000, n_tokens=24, n_ctx=64, seed=19, qkv_bias=True, tied=False)


# one query head per KV head, and 12 per KV head (two head blocks, the second one partly filled)
TINY_MHA = synth.ModelConfig(name="tiny_mha", n_layers=2, hidden=128, n_head=4, n_head_kv=4, head_dim=64,
                             ffn=256, vocab=1000, n_tokens=20, n_ctx=80, seed=23, qkv_bias=True, tied=True)
TINY_G12 = synth.ModelConfig(name="tiny_gqa12", n_layers=2, hidden=256, n_head=24, n_head_kv=2, head_dim=128,
                             ffn=384, vocab=1000, n_tokens=20, n_ctx=80, seed=29, qkv_bias=False, qk_norm=True,
                             tied=False)


@pytest.mark.parametrize("cfg", [synth.LAYER1, TINY_Q3, TINY_Q2, TINY_WIDE, TINY_MHA, TINY_G12],
                         ids=lambda c: c.name)
def test_decode_matches_oracle(cfg):
    """Head dims 64 and 128, QKV bias, per-head QK norm, tied and separate lm_heads, GQA 7:1, 4:1,
    4:1 with one KV head, 5:1, 1:1 and 12:1, an attention row wider than the hidden size (40 x 128
    over 256); several steps, each attending to the prompt and the earlier steps."""
    dev = need_gpu()
    m, steps, kk, vv, end = prefill_then_decode(cfg, dev, 4)
    for i, (got, want) in enumerate(steps):
        compare_logits(got, want, f"{cfg.name} step {i} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"{cfg.name} step {i} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert np.all(gk[:, end:] == SENTINEL) and np.all(gv[:, end:] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, :end], kk[:, :end], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, :end], vv[:, :end], max_ulp=64, max_frac_inexact=0.05, what="V regions")


# random small models (other draws than the forward's), each with room for its decode steps
RANDOM_DECODE = [c for c, _ in _random_tiny_configs(8, 20261207) if c.n_ctx >= c.prefix_tokens + c.n_tokens + 3]


@pytest.mark.parametrize("cfg", RANDOM_DECODE,
                         ids=[f"{c.name}_L{c.n_layers}_h{c.hidden}_{c.n_head}x{c.head_dim}_kv{c.n_head_kv}"
                              f"_f{c.ffn}_t{c.n_tokens}_p{c.prefix_tokens}_ctx{c.n_ctx}" for c in RANDOM_DECODE])
def test_decode_random_small_models_match_oracle(cfg):
    """Three decode steps after the prompt of a random small model, every step's logits and the
    regions against the oracle."""
    dev = need_gpu()
    m, steps, kk, vv, end = prefill_then_decode(cfg, dev, 3)
    for i, (got, want) in enumerate(steps):
        compare_logits(got, want, f"{cfg.name} step {i} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"{cfg.name} step {i} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert np.all(gk[:, end:] == SENTINEL) and np.all(gv[:, end:] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, :end], kk[:, :end], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, :end], vv[:, :end], max_ulp=64, max_frac_inexact=0.05, what="V regions")


def test_decode_graph_replays_at_new_positions():
    """One captured decode step replayed at successive positions (the position is staged per launch)
    computes what the eager steps compute."""
    dev = need_gpu()
    cfg = TINY_Q3
    _, steps, _, _, _ = prefill_then_decode(cfg, dev, 5, graph=True)
    for i, (got, want) in enumerate(steps):
        compare_logits(got, want, f"graph step {i} logits")


def test_decode_equals_prefill_of_one_token():
    """mi_decode_step and mi_prefill_forward with one token are the same call (bit for bit), and a
    decode step after a prefill equals the last row of a prefill of prompt + token."""
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    n = cfg.n_tokens
    pos = np.arange(n, dtype=np.int32)
    full = m.forward(ids, pos).cpu().numpy().copy()         # prompt of n tokens at once
    m.kv_k.fill_(SENTINEL)
    m.kv_v.fill_(SENTINEL)
    m.forward(ids[:n - 1], pos[:n - 1])
    a = m.decode(int(ids[n - 1]), n - 1).cpu().numpy().copy()
    b = m.forward(ids[n - 1:], pos[n - 1:]).cpu().numpy().copy()
    np.testing.assert_array_equal(a, b)
    assert_f32_match(a, full, max_ulp=4, max_frac_inexact=0.01, what="decode vs one-shot prefill")


def test_decode_argument_errors_leave_state_untouched():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    before = m.kv_k.cpu().numpy().copy()
    with pytest.raises(B.MiError) as e:
        m.decode(1, cfg.n_ctx)
    assert e.value.code == B.MI_ERR_POSITION_RANGE
    with pytest.raises(B.MiError) as e:
        m.decode(cfg.vocab, 0)
    assert e.value.code == B.MI_ERR_INVALID_ARG
    torch.cuda.synchronize()
    np.testing.assert_array_equal(m.kv_k.cpu().numpy(), before)


def test_headline_config_decode_matches_oracle():
    """The 24-layer 0.5B-shaped model: the 512-token prompt, then 3 decode steps at 512..514."""
    dev = need_gpu()
    cfg = synth.QWEN2_0P5B
    m, steps, kk, vv, end = prefill_then_decode(cfg, dev, 3)
    for i, (got, want) in enumerate(steps):
        compare_logits(got, want, f"{cfg.name} step {i} logits")
    gk = m.kv_k.cpu().numpy()
    d = np.linalg.norm(gk[:, :end] - kk[:, :end]) / np.linalg.norm(kk[:, :end])
    say(f"  K regions rel-L2 {d:.3e}, identical {np.mean(gk[:, :end] == kk[:, :end]):.6f}")
    assert d <= 1e-3 and np.all(gk[:, end:] == SENTINEL)


# head_dim 128 with keys spread over several of the one-token attention's key ranges (64 keys each
# for n_ctx 800): the last prompt token sits at position 599, so its attention merges ten ranges
TINY_Q3_LONG = synth.ModelConfig(name="tiny_qwen3_long", n_layers=2, hidden=256, n_head=4, n_head_kv=2,
                                 head_dim=128, ffn=384, vocab=1000, n_tokens=40, n_ctx=800, seed=17,
                                 qkv_bias=False, qk_norm=True, tied=True, prefix_tokens=560)


def test_one_token_tail_merges_key_ranges_head_dim_128():
    """The last prompt token of a prefill (n_out = 1) and the decode steps after it run the
    one-token attention, whose key ranges are merged by one more kernel: with head_dim 128 and
    positions past 512 several ranges carry keys.  Logits and regions against the
    oracle, for the prefill and for 3 decode steps at 600..602."""
    dev = need_gpu()
    cfg = TINY_Q3_LONG
    m, w = load_pair(cfg, dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    m.forward(pre_ids, pre_pos)
    oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
    got = m.forward(ids, pos).cpu().numpy()
    want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
    compare_logits(got, want, f"{cfg.name} prefill logits (last position {int(pos[-1])})")
    assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what="prefill logits ulp")
    for i, tok in enumerate(decode_tokens(cfg, 3)):
        p = int(pos[-1]) + 1 + i
        say(f"decode {cfg.name} step {i} position {p}")
        got = m.decode(int(tok), p).cpu().numpy().copy()
        want = oracle.prefill_forward(cfg, w, np.array([tok], np.int32), np.array([p], np.int32), cfg.n_ctx, kk, vv)[0]
        compare_logits(got, want, f"{cfg.name} step {i} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"step {i} logits ulp")
    end = int(pos[-1]) + 4
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert np.all(gk[:, end:] == SENTINEL) and np.all(gv[:, end:] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, :end], kk[:, :end], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, :end], vv[:, :end], max_ulp=64, max_frac_inexact=0.05, what="V regions")


# n_ctx above 4096: the one-token attention's key ranges grow to 128 keys, two sub-chunks of 64
# (40 ranges for 5120)
TINY_FAR = synth.ModelConfig(name="tiny_far_positions", n_layers=2, hidden=128, n_head=4, n_head_kv=2, head_dim=64,
                             ffn=192, vocab=700, n_tokens=20, n_ctx=5120, seed=23, qkv_bias=True)
TINY_FAR_Q3 = synth.ModelConfig(name="tiny_far_qwen3", n_layers=2, hidden=256, n_head=8, n_head_kv=2, head_dim=128,
                                ffn=384, vocab=700, n_tokens=20, n_ctx=5120, seed=31, qkv_bias=False, qk_norm=True,
                                tied=False)


@pytest.mark.parametrize("cfg", [TINY_FAR, TINY_FAR_Q3], ids=lambda c: c.name)
def test_far_positions_over_long_context(cfg):
    """A prompt at positions 5040..5059 of a 5120-row context (the rows below it hold the regions'
    fill, read by both sides), then 3 decode steps: every key range of 128 keys carries keys, the
    range holding the position (4992..) spans two sub-chunks, and the merge combines 40 ranges.  Head dims
    64 and 128 (with the QK norm).  Logits and regions against the oracle."""
    dev = need_gpu()
    m, w = load_pair(cfg, dev, max_tokens=cfg.n_tokens)
    _, ids = synth.gen_token_ids(cfg)
    pos = np.arange(5040, 5040 + cfg.n_tokens, dtype=np.int32)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    got = m.forward(ids, pos).cpu().numpy().copy()
    want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
    compare_logits(got, want, f"{cfg.name} prefill logits")
    for i, tok in enumerate(decode_tokens(cfg, 3)):
        p = int(pos[-1]) + 1 + i
        say(f"decode {cfg.name} step {i} position {p}")
        got = m.decode(int(tok), p).cpu().numpy().copy()
        want = oracle.prefill_forward(cfg, w, np.array([tok], np.int32), np.array([p], np.int32), cfg.n_ctx, kk, vv)[0]
        compare_logits(got, want, f"{cfg.name} step {i} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"step {i} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert_f32_match(gk, kk, max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv, vv, max_ulp=64, max_frac_inexact=0.05, what="V regions")


def test_decode_at_first_and_last_rows():
    """A decode step as the very first token (position 0: one key, one range) and at the last row
    of the context (position n_ctx - 1), each against the oracle's one-token forward."""
    dev = need_gpu()
    cfg = TINY_Q3
    m, w = load_pair(cfg, dev)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    for tok, p in zip(decode_tokens(cfg, 2), [0, cfg.n_ctx - 1]):
        say(f"decode {cfg.name} token {int(tok)} at position {p}")
        got = m.decode(int(tok), p).cpu().numpy().copy()
        want = oracle.prefill_forward(cfg, w, np.array([tok], np.int32), np.array([p], np.int32), cfg.n_ctx, kk, vv)[0]
        compare_logits(got, want, f"position {p} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"position {p} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert_f32_match(gk, kk, max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv, vv, max_ulp=64, max_frac_inexact=0.05, what="V regions")


def test_back_to_back_steps_through_the_stage_ring():
    """Ten decode steps enqueued without a host synchronization between them (more than the stage's
    four pinned buffers, each read on the device by the first kernel of its call): the regions and
    each step's logits (copied to a buffer of its own) equal the oracle's steps."""
    dev = need_gpu()
    cfg = TINY_Q3
    m, w = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    n = 12
    pos = np.arange(n, dtype=np.int32)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    m.forward(ids[:n], pos)
    oracle.prefill_forward(cfg, w, ids[:n], pos, cfg.n_ctx, kk, vv)
    toks = decode_tokens(cfg, 10)
    outs = [torch.empty(cfg.vocab, dtype=torch.float32, device=dev) for _ in toks]
    for i, tok in enumerate(toks):  # no synchronization in between
        m.decode(int(tok), n + i, logits=outs[i])
    torch.cuda.synchronize()
    for i, tok in enumerate(toks):
        want = oracle.prefill_forward(cfg, w, np.array([tok], np.int32), np.array([n + i], np.int32), cfg.n_ctx,
                                      kk, vv)[0]
        compare_logits(outs[i].cpu().numpy(), want, f"back-to-back step {i}")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    end = n + len(toks)
    assert np.all(gk[:, end:] == SENTINEL) and np.all(gv[:, end:] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, :end], kk[:, :end], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, :end], vv[:, :end], max_ulp=64, max_frac_inexact=0.05, what="V regions")

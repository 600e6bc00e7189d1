"""End-to-end parity of mi_prefill_forward with the oracle, plus the forward's invariants on GPU."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_transformer_prefill_amd import binding as B
from quantized_transformer_prefill_amd.model import PrefillModel
from tests.gpu_util import assert_f32_match, need_gpu, say

pytestmark = pytest.mark.gpu

SENTINEL = -777.25

# the bar for last-token logits (max-abs and rel-L2 against the oracle)
MAX_ABS, REL_L2 = 2e-2, 1e-3


def load_pair(cfg, dev, max_tokens=None, kv_fill=SENTINEL):
    """GPU model and oracle weights from the same seeded draws (drawn once, on the device)."""
    host = {}

    def tensors():
        for name, kind, t in synth.iter_tensors(cfg, device=dev):
            host[name] = t.cpu().numpy()
            yield name, kind, t

    m = PrefillModel(cfg, tensors(), max_tokens or cfg.prefix_tokens + cfg.n_tokens, cfg.n_ctx, device=dev,
                     kv_fill=kv_fill)
    q8 = [n for n, s, k in synth.tensor_specs(cfg) if k == "q8"]
    return m, oracle.weights_from_arrays(host, q8)


def compare_logits(got, want, what):
    got = np.asarray(got, np.float32)
    d = got.astype(np.float64) - want
    rel = np.linalg.norm(d) / np.linalg.norm(want)
    say(f"  {what}: max-abs {np.abs(d).max():.3e} rel-L2 {rel:.3e} identical {np.mean(got == want):.6f}")
    assert np.abs(d).max() <= MAX_ABS and rel <= REL_L2, what


def run_pair(cfg, dev):
    m, w = load_pair(cfg, dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    if cfg.prefix_tokens:
        m.forward(pre_ids, pre_pos)
        oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
    logits = m.forward(ids, pos).cpu().numpy()
    want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
    return m, logits, want, kk, vv


TINY_Q3 = synth.ModelConfig(name="tiny_qwen3", n_layers=3, hidden=256, n_head=8, n_head_kv=2, head_dim=128,
                            ffn=384, vocab=1000, n_tokens=45, n_ctx=96, seed=7, qkv_bias=False, qk_norm=True,
                            tied=True)
TINY_Q2 = synth.ModelConfig(name="tiny_qwen2_ctx", n_layers=2, hidden=128, n_head=4, n_head_kv=1, head_dim=64,
                            ffn=192, vocab=700, n_tokens=20, n_ctx=50, seed=8, qkv_bias=True, prefix_tokens=17)


@pytest.mark.parametrize("cfg", [synth.LAYER1, TINY_Q3, TINY_Q2], ids=lambda c: c.name)
def test_forward_matches_oracle(cfg):
    dev = need_gpu()
    say(f"forward {cfg.name}")
    m, logits, want, kk, vv = run_pair(cfg, dev)
    compare_logits(logits, want, f"{cfg.name} logits")
    assert_f32_match(logits, want, max_ulp=64, max_frac_inexact=0.05, what=f"{cfg.name} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    used = np.arange(cfg.prefix_tokens + cfg.n_tokens)
    free = np.arange(used.size, cfg.n_ctx)
    assert np.all(gk[:, free] == SENTINEL) and np.all(gv[:, free] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, used], kk[:, used], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, used], vv[:, used], max_ulp=64, max_frac_inexact=0.05, what="V regions")


@pytest.mark.parametrize("cfg,n_outs", [(synth.LAYER1, (1, 3, 16)), (TINY_Q3, (2, 45)), (TINY_Q2, (20,))],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_forward_n_out_matches_oracle(cfg, n_outs):
    """Logits of the last n_out tokens (the tail rows of the last layer), against the oracle."""
    dev = need_gpu()
    m, w = load_pair(cfg, dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    for n_out in n_outs:
        say(f"forward_n {cfg.name} n_out={n_out}")
        m.kv_k.fill_(SENTINEL)
        m.kv_v.fill_(SENTINEL)
        kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
        if cfg.prefix_tokens:
            m.forward(pre_ids, pre_pos)
            oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
        got = m.forward_n(ids, pos, n_out).cpu().numpy()
        want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv, n_out=n_out)
        assert got.shape == want.shape == (n_out, cfg.vocab)
        compare_logits(got, want, f"{cfg.name} n_out={n_out} logits")
        assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"{cfg.name} n_out={n_out} ulp")
        one = m.forward(ids, pos).cpu().numpy()
        np.testing.assert_array_equal(got[-1], one)   # the last row is the n_out = 1 logits


def _random_tiny_configs(n_cases, seed):
    """Seeded random small models: 1-3 layers, hidden 64..512, head layouts with GQA groups of 1-8 at
    head_dim 64 or 128, ffn 64..640, with or without Q/K/V bias and per-head QK norm, tied or separate
    lm_head, a prompt of 1-80 tokens after a prefix of 0-30, n_ctx up to 200 rows; plus an n_out (1 in
    about half the cases: the last layer's one-token tail)."""
    rng = np.random.default_rng(seed)
    layouts = [(4, 1), (4, 2), (4, 4), (8, 2), (8, 1), (6, 3)]
    out = []
    for i in range(n_cases):
        nh, nkv = layouts[int(rng.integers(len(layouts)))]
        n_tokens = int(rng.integers(1, 81))
        prefix = int(rng.choice([0, 0, int(rng.integers(1, 31))]))
        cfg = synth.ModelConfig(
            name=f"rand{i}", n_layers=int(rng.integers(1, 4)), hidden=32 * int(rng.integers(2, 17)),
            n_head=nh, n_head_kv=nkv, head_dim=int(rng.choice([64, 128])), ffn=32 * int(rng.integers(2, 21)),
            vocab=int(rng.integers(200, 1500)), n_tokens=n_tokens,
            n_ctx=prefix + n_tokens + int(rng.integers(0, 201 - n_tokens)), seed=int(rng.integers(1000)),
            qkv_bias=bool(rng.integers(2)), qk_norm=bool(rng.integers(2)), tied=bool(rng.integers(2)),
            prefix_tokens=prefix)
        out.append((cfg, 1 if rng.integers(2) else int(rng.integers(1, n_tokens + 1))))
    return out


RANDOM_TINY = _random_tiny_configs(12, 20261206)


@pytest.mark.parametrize("cfg,n_out", RANDOM_TINY,
                         ids=[f"{c.name}_L{c.n_layers}_h{c.hidden}_{c.n_head}x{c.head_dim}_kv{c.n_head_kv}"
                              f"_f{c.ffn}_t{c.n_tokens}_p{c.prefix_tokens}_o{o}" for c, o in RANDOM_TINY])
def test_random_small_models_match_oracle(cfg, n_out):
    """Whole forwards of random small models: the last n_out logits and every K/V region row against
    the oracle, and nothing written past the prompt's rows."""
    dev = need_gpu()
    say(f"random forward {cfg}")
    m, w = load_pair(cfg, dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
    if cfg.prefix_tokens:
        m.forward(pre_ids, pre_pos)
        oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
    got = m.forward_n(ids, pos, n_out).cpu().numpy()
    want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv, n_out=n_out)
    compare_logits(got, want, f"{cfg.name} n_out={n_out} logits")
    assert_f32_match(got, want, max_ulp=64, max_frac_inexact=0.05, what=f"{cfg.name} logits ulp")
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    used = np.arange(cfg.prefix_tokens + cfg.n_tokens)
    free = np.arange(used.size, cfg.n_ctx)
    assert np.all(gk[:, free] == SENTINEL) and np.all(gv[:, free] == SENTINEL), "stray KV writes"
    assert_f32_match(gk[:, used], kk[:, used], max_ulp=64, max_frac_inexact=0.05, what="K regions")
    assert_f32_match(gv[:, used], vv[:, used], max_ulp=64, max_frac_inexact=0.05, what="V regions")


def test_forward_n_out_bounds():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    pos = np.arange(cfg.n_tokens, dtype=np.int32)
    for bad in (0, cfg.n_tokens + 1):
        with pytest.raises(B.MiError) as e:
            m.forward_n(ids, pos, bad)
        assert e.value.code == B.MI_ERR_INVALID_ARG


def _reset(m):
    m.kv_k.fill_(SENTINEL)
    m.kv_v.fill_(SENTINEL)


@pytest.mark.parametrize("cfg,n_out", [(synth.LAYER1, 1), (TINY_Q3, 3), (TINY_Q2, 1)], ids=lambda v: getattr(v, "name", str(v)))
def test_graph_replay_equals_eager(cfg, n_out):
    """The captured forward, replayed several times with eager work and synchronizations in between,
    gives bit-identical logits and KV rows to the eager call on the same ids and positions --
    including positions that differ between replays (the largest position is staged per launch)."""
    dev = need_gpu()
    m, _ = load_pair(cfg, dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    nt = cfg.n_tokens
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = m.graph(nt, n_out)
        assert g.nodes() >= 2 + 5 * cfg.n_layers   # embedding, >= 5 kernels per layer, the head
        shifts = [0, 3, 0] if cfg.prefix_tokens == 0 else [0, 0]
        for r, shift in enumerate(shifts):
            say(f"graph {cfg.name} replay {r} shift {shift}")
            p = pos + shift
            _reset(m)
            if cfg.prefix_tokens:
                m.forward(pre_ids, pre_pos)
            eager = m.forward_n(ids, p, n_out).cpu().numpy().copy()
            k_eager = m.kv_k.cpu().numpy().copy()
            _reset(m)
            if cfg.prefix_tokens:
                m.forward(pre_ids, pre_pos)
            got = g.launch(ids, p).cpu().numpy().copy()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got, eager)
            np.testing.assert_array_equal(m.kv_k.cpu().numpy(), k_eager)
            _ = torch.ones(1000, device=dev).sum().item()   # unrelated eager work between replays
        with pytest.raises(B.MiError) as e:
            g.launch(ids, np.zeros(nt, dtype=np.int32))
        assert e.value.code == B.MI_ERR_DUP_POSITION
        g.close()


def test_prefill_equals_replay_and_chunks_on_gpu():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    pos = np.arange(cfg.n_tokens, dtype=np.int32)
    full = m.forward(ids, pos).cpu().numpy().copy()
    k_full = m.kv_k.cpu().numpy().copy()
    m.kv_k.fill_(SENTINEL)
    m.kv_v.fill_(SENTINEL)
    for t in range(cfg.n_tokens):                       # token by token through the same regions
        step = m.forward(ids[t:t + 1], pos[t:t + 1]).cpu().numpy().copy()
    assert_f32_match(step, full, max_ulp=4, max_frac_inexact=0.01, what="replay logits")
    assert_f32_match(m.kv_k.cpu().numpy(), k_full, max_ulp=4, max_frac_inexact=0.01, what="replay K")
    m.kv_k.fill_(SENTINEL)
    m.kv_v.fill_(SENTINEL)
    m.forward(ids[:5], pos[:5])                         # prefix, then the rest at later positions
    two = m.forward(ids[5:], pos[5:]).cpu().numpy().copy()
    assert_f32_match(two, full, max_ulp=4, max_frac_inexact=0.01, what="chunked logits")


TINY_PERM = synth.ModelConfig(name="tiny_qwen2_perm", n_layers=2, hidden=128, n_head=4, n_head_kv=1, head_dim=64,
                              ffn=192, vocab=700, n_tokens=37, n_ctx=64, seed=9, qkv_bias=True)


def test_forward_positions_out_of_order_match_oracle():
    """Positions are data (a token at position p attends to region rows 0..p after this call's
    stores): 37 tokens given out of order with gaps, the largest position n_ctx - 1 on a middle
    token and not on the last one, whose logits are returned (row nt - 1).  Rows the call does not
    write keep what the caller left there (zeros) and are read as such by later positions."""
    dev = need_gpu()
    cfg = TINY_PERM
    m, w = load_pair(cfg, dev, kv_fill=0.0)
    _, ids = synth.gen_token_ids(cfg)
    rng = np.random.default_rng(11)
    pos = rng.choice(cfg.n_ctx - 1, cfg.n_tokens, replace=False).astype(np.int32)
    pos[cfg.n_tokens // 2] = cfg.n_ctx - 1
    say(f"forward {cfg.name}: positions {pos.tolist()}")
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=0.0)
    got = m.forward(ids, pos).cpu().numpy()
    want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
    compare_logits(got, want, f"{cfg.name} logits")
    written = np.zeros(cfg.n_ctx, dtype=bool)
    written[pos] = True
    gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
    assert np.all(gk[:, ~written] == 0) and np.all(gv[:, ~written] == 0)
    for name, g, o in (("K", gk, kk), ("V", gv, vv)):
        d = np.linalg.norm(g[:, written] - o[:, written]) / np.linalg.norm(o[:, written])
        say(f"  {name} rows rel-L2 {d:.3e}")
        assert d <= 1e-3


def test_future_tokens_leave_earlier_kv_rows_bit_identical():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    pos = np.arange(cfg.n_tokens, dtype=np.int32)
    m.forward(ids, pos)
    k1 = m.kv_k.cpu().numpy().copy()
    ids2 = ids.copy()
    ids2[10:] = (ids2[10:] + 1) % cfg.vocab
    m.forward(ids2, pos)
    k2 = m.kv_k.cpu().numpy()
    np.testing.assert_array_equal(k1[:, :10], k2[:, :10])
    assert not np.array_equal(k1[:, 10:16], k2[:, 10:16])


def test_forward_errors_leave_state_untouched():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    before = m.kv_k.cpu().numpy().copy()
    with pytest.raises(B.MiError) as e:
        m.forward([1, 2], [0, cfg.n_ctx])
    assert e.value.code == B.MI_ERR_POSITION_RANGE
    with pytest.raises(B.MiError) as e:
        m.forward([1, 2], [3, 3])
    assert e.value.code == B.MI_ERR_DUP_POSITION
    torch.cuda.synchronize()
    np.testing.assert_array_equal(m.kv_k.cpu().numpy(), before)


def test_headline_config_matches_oracle():
    """The 24-layer 0.5B-shaped model on its 512-token prompt: logits, and the K and V rows of every
    layer, against the oracle."""
    dev = need_gpu()
    cfg = synth.QWEN2_0P5B
    say(f"forward {cfg.name}")
    m, logits, want, kk, vv = run_pair(cfg, dev)
    compare_logits(logits, want, f"{cfg.name} logits")
    compare_regions(m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy(), kk, vv, cfg.n_tokens, cfg.name)


def compare_regions(gk, gv, kk, vv, used, what):
    """K and V regions of every layer (host copies): rows 0..used-1 against the oracle's (f32 values
    rounded from f64 node results: identical but for rare one-ulp f64 ties), rows past them untouched."""
    for name, g, o in (("K", gk, kk), ("V", gv, vv)):
        assert np.all(g[:, used:] == SENTINEL), f"{what}: stray {name} writes"
        d = np.linalg.norm(g[:, :used] - o[:, :used]) / np.linalg.norm(o[:, :used])
        say(f"  {what} {name} regions rel-L2 {d:.3e}")
        assert_f32_match(g[:, :used], o[:, :used], max_ulp=64, max_frac_inexact=1e-3, what=f"{what} {name} regions")


@pytest.mark.parametrize("name", ["qwen2p5_7b_pp2048", "qwen3_8b_chunk3072at1024"])
def test_large_configs_full_size_properties(name):
    """The 7B- and 8B-shaped configurations at full size, in the launch configuration the bench
    times (eager call and captured-graph replay), checked by properties that hold at any size (their
    oracle comparison, minutes of host time, is test_zx_full_size_gpu.py, collected last):
    a repeated call and the graph replay give bit-identical logits and KV regions; rows no call
    wrote keep their sentinel; logits are finite; changing only the last token leaves every KV row
    at an earlier position bit-identical in every layer, and changes the last position's K row."""
    dev = need_gpu()
    cfg = synth.MODEL_CONFIGS[name]
    say(f"properties {cfg.name}: loading")
    m = PrefillModel(cfg, synth.iter_tensors(cfg, device=dev), cfg.prefix_tokens + cfg.n_tokens, cfg.n_ctx,
                     device=dev, kv_fill=SENTINEL)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    if cfg.prefix_tokens:
        m.forward(pre_ids, pre_pos)
    say(f"  eager call x2")
    l1 = m.forward(ids, pos).clone()
    k1, v1 = m.kv_k.clone(), m.kv_v.clone()
    l2 = m.forward(ids, pos).clone()
    assert torch.equal(l1, l2) and torch.equal(m.kv_k, k1) and torch.equal(m.kv_v, v1)
    assert bool(torch.isfinite(l1).all())
    used = int(pos.max()) + 1
    assert bool((k1[:, used:] == SENTINEL).all()) and bool((v1[:, used:] == SENTINEL).all())
    assert not bool((k1[:, :used] == SENTINEL).any())
    say(f"  graph replay")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = m.graph(cfg.n_tokens)
        l3 = g.launch(ids, pos).clone()
        torch.cuda.synchronize()
        g.close()
    assert torch.equal(l1.reshape(-1), l3.reshape(-1)) and torch.equal(m.kv_k, k1) and torch.equal(m.kv_v, v1)
    say(f"  last token changed")
    ids2 = ids.copy()
    ids2[-1] = (ids2[-1] + 1) % cfg.vocab
    l4 = m.forward(ids2, pos)
    last = int(pos[-1])
    assert torch.equal(m.kv_k[:, :last], k1[:, :last]) and torch.equal(m.kv_v[:, :last], v1[:, :last])
    assert not torch.equal(m.kv_k[0, last], k1[0, last])
    assert not torch.equal(l4, l1)

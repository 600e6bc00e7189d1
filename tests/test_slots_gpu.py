"""mi_prefill_forward_slots: several sequences, each with its own regions and positions, in one call,
against the oracle's prefill of each sequence alone over its own regions."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_transformer_prefill_amd import binding as B
from tests.gpu_util import assert_f32_match, need_gpu, say
from tests.test_forward_gpu import SENTINEL, TINY_Q3, _random_tiny_configs, compare_logits, load_pair

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [synth.LAYER1, TINY_Q3], ids=lambda c: c.name)
def test_slots_match_independent_oracle_calls(cfg):
    dev = need_gpu()
    m, w = load_pair(cfg, dev, max_tokens=48)
    rng = np.random.default_rng(cfg.seed + 77)
    # slot 0: 20 fresh tokens at 0..19 (two query tiles, the second ragged); slot 1: a 10-token prefix (own call), then 5 tokens at 10..14;
    # slot 2: 16 tokens at 0..15 in the model's own regions; slot 3: 1 token at 3 (rows 0..2 unwritten)
    sets = [m.new_kv_set(SENTINEL), m.new_kv_set(SENTINEL), m.own_kv_set(), m.new_kv_set(SENTINEL)]
    okv = [oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL) for _ in sets]
    pre_ids = rng.integers(0, cfg.vocab, 10).astype(np.int32)
    m.forward_slots([(pre_ids, np.arange(10, dtype=np.int32), sets[1])])
    oracle.prefill_forward(cfg, w, pre_ids, np.arange(10, dtype=np.int32), cfg.n_ctx, *okv[1])
    slots = [
        (rng.integers(0, cfg.vocab, 20).astype(np.int32), np.arange(20, dtype=np.int32)),
        (rng.integers(0, cfg.vocab, 5).astype(np.int32), np.arange(10, 15, dtype=np.int32)),
        (rng.integers(0, cfg.vocab, 16).astype(np.int32), rng.permutation(16).astype(np.int32)),
        (rng.integers(0, cfg.vocab, 1).astype(np.int32), np.array([3], np.int32)),
    ]
    got = m.forward_slots([(a, b, ks) for (a, b), ks in zip(slots, sets)]).cpu().numpy()
    for i, ((ids, pos), ks, (kk, vv)) in enumerate(zip(slots, sets, okv)):
        want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
        compare_logits(got[i], want, f"{cfg.name} slot {i} logits")
        assert_f32_match(got[i], want, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} logits ulp")
        gk, gv = ks.k.cpu().numpy(), ks.v.cpu().numpy()
        assert_f32_match(gk, kk, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} K regions")
        assert_f32_match(gv, vv, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} V regions")


RANDOM_SLOT_MODELS = [c for c, _ in _random_tiny_configs(4, 20261208)]


@pytest.mark.parametrize("cfg", RANDOM_SLOT_MODELS,
                         ids=[f"{c.name}_L{c.n_layers}_h{c.hidden}_{c.n_head}x{c.head_dim}_kv{c.n_head_kv}_ctx{c.n_ctx}"
                              for c in RANDOM_SLOT_MODELS])
def test_slots_random_match_independent_oracle_calls(cfg):
    """2-6 sequences of random lengths, each a run of positions at a random offset in its own
    regions (the rows before the run are unwritten), against the oracle's prefill of each alone."""
    dev = need_gpu()
    rng = np.random.default_rng(cfg.seed + 99)
    n_slots = int(rng.integers(2, 7))
    lens = [min(int(rng.integers(1, 25)), cfg.n_ctx) for _ in range(n_slots)]
    say(f"slots {cfg.name}: lengths {lens}")
    m, w = load_pair(cfg, dev, max_tokens=sum(lens))
    sets = [m.new_kv_set(SENTINEL) for _ in range(n_slots)]
    okv = [oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL) for _ in sets]
    slots = []
    for n in lens:
        start = int(rng.integers(0, cfg.n_ctx - n + 1))
        slots.append((rng.integers(0, cfg.vocab, n).astype(np.int32), (start + np.arange(n)).astype(np.int32)))
    got = m.forward_slots([(a, b, ks) for (a, b), ks in zip(slots, sets)]).cpu().numpy()
    for i, ((ids, pos), ks, (kk, vv)) in enumerate(zip(slots, sets, okv)):
        want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)[0]
        compare_logits(got[i], want, f"{cfg.name} slot {i} logits")
        assert_f32_match(got[i], want, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} logits ulp")
        assert_f32_match(ks.k.cpu().numpy(), kk, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} K regions")
        assert_f32_match(ks.v.cpu().numpy(), vv, max_ulp=64, max_frac_inexact=0.05, what=f"slot {i} V regions")


def test_one_slot_equals_forward():
    """One slot in the model's own regions is the plain forward, bit for bit (logits and regions)."""
    dev = need_gpu()
    cfg = TINY_Q3
    m, _ = load_pair(cfg, dev)
    _, ids = synth.gen_token_ids(cfg)
    pos = np.arange(ids.size, dtype=np.int32)
    a = m.forward(ids, pos).cpu().numpy().copy()
    ka = m.kv_k.cpu().numpy().copy()
    m.kv_k.fill_(SENTINEL)
    m.kv_v.fill_(SENTINEL)
    b = m.forward_slots([(ids, pos, m.own_kv_set())]).cpu().numpy()[0]
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(ka, m.kv_k.cpu().numpy())


def test_slots_argument_errors_write_nothing():
    dev = need_gpu()
    cfg = synth.LAYER1
    m, _ = load_pair(cfg, dev)
    a, b = m.new_kv_set(SENTINEL), m.own_kv_set()
    before = b.k.cpu().numpy().copy()
    with pytest.raises(B.MiError) as e:   # position repeated inside a slot
        m.forward_slots([([1, 2], [0, 1], a), ([3, 4], [5, 5], b)])
    assert e.value.code == B.MI_ERR_DUP_POSITION
    with pytest.raises(B.MiError) as e:   # too many tokens for the workspace
        m.forward_slots([([1] * cfg.n_tokens, list(range(cfg.n_tokens)), a), ([2], [0], b)])
    assert e.value.code == B.MI_ERR_WORKSPACE
    torch.cuda.synchronize()
    np.testing.assert_array_equal(b.k.cpu().numpy(), before)
    assert np.all(a.k.cpu().numpy() == SENTINEL)

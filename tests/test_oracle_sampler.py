"""Pins of the oracle sampler against facts fixed outside its code: the published SplitMix64
sequence, hand-computed penalty values, closed forms (greedy = argmax), the step order the pages
give (top-p before temperature), and sampling frequencies against the exact distribution."""
import math

import numpy as np

from oracle import sampler as S


def test_splitmix64_published_sequence():
    # the generator seeded with 0: outputs published with the reference implementation
    assert [S.splitmix64(0, i) for i in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_uniform_range_and_moments():
    u = np.array([S.uniform(12345, i) for i in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1.0 / 12.0) < 0.005


def test_penalties_hand_example():
    p = S.SamplerParams(repeat_penalty=2.0, frequency_penalty=0.5, presence_penalty=0.25)
    out = S.penalize([2.0, -1.0, 0.5, 3.0], [0, 1, 1, 3], p)
    # t0: 2/2 - 0.5 - 0.25; t1: -1*2 - 2*0.5 - 0.25; t2 untouched; t3: 3/2 - 0.5 - 0.25
    np.testing.assert_array_equal(out, [0.25, -3.25, 0.5, 0.75])


def test_window_is_the_last_64_tokens():
    p = S.SamplerParams(presence_penalty=1.0)
    window = [5] + [7] * 64          # token 5 fell out of the window
    out = S.penalize(np.zeros(8), window, p)
    assert out[5] == 0.0 and out[7] == -1.0


def test_greedy_and_top1_are_the_argmax_with_smallest_id_on_ties():
    logits = np.array([0.5, 2.0, 2.0, -1.0], np.float32)
    for step in range(20):
        assert S.sample(logits, [], S.SamplerParams(temperature=0.0), 1, step) == 1
        assert S.sample(logits, [], S.SamplerParams(top_k=1), 1, step) == 1


def test_top_p_uses_the_untempered_distribution():
    # untempered: p0 = e/(e+1) = 0.731 >= 0.7 -> only token 0 survives, whatever the temperature;
    # tempering first (T = 10) would give p0 = 0.525 and keep both
    p = S.SamplerParams(top_k=2, top_p=0.7, temperature=10.0)
    assert {S.sample([1.0, 0.0], [], p, 3, i) for i in range(200)} == {0}


def test_frequencies_match_the_tempered_softmax():
    logits = np.array([1.0, 0.2, -0.5, 0.9, -2.0, 0.0], np.float32)
    T, n = 0.7, 30000
    p = S.SamplerParams(top_k=6, temperature=T)
    counts = np.bincount([S.sample(logits, [], p, 99, i) for i in range(n)], minlength=6)
    w = np.exp(logits.astype(np.float64) / T)
    want = w / w.sum()
    se = np.sqrt(want * (1 - want) / n)
    assert np.all(np.abs(counts / n - want) < 5 * se + 1e-12), (counts / n, want)


def test_top_k_and_top_p_restrict_the_support():
    logits = np.array([3.0, 2.9, 1.0, 0.5, 0.4], np.float32)
    seen = {S.sample(logits, [], S.SamplerParams(top_k=2), 5, i) for i in range(500)}
    assert seen == {0, 1}
    # probabilities of the 5: 0.44, 0.40, 0.06, ...; top_p 0.8 keeps the first two
    w = np.exp(logits - logits[0]); prob = w / w.sum()
    assert prob[0] < 0.8 <= prob[0] + prob[1]
    seen = {S.sample(logits, [], S.SamplerParams(top_k=5, top_p=0.8), 6, i) for i in range(500)}
    assert seen == {0, 1}

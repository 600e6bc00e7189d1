"""Oracle sampler: one next token from last-token logits (TEST INFRASTRUCTURE ONLY).

The index of the walkthrough names the sampler's chain (its row for doc 12): penalties over a
window of the last 64 tokens (repeat, frequency, presence) -> top-k -> top-p -> temperature ->
seeded sample.  The pages name the steps and their order, not their formulas; this module takes
the plainest reading of each step:

  penalties   for a token t seen c_t > 0 times in the window, in f64 from its f32 logit:
                  l = l / repeat if l > 0 else l * repeat
                  l = l - c_t * frequency - presence
              tokens outside the window keep their logit (as f64)
  top-k       the k largest penalized logits, ties broken by the smaller token id
  top-p       softmax of the k candidates (the untempered logits: temperature comes later in
              the chain); keep the shortest prefix, in the order above, whose cumulative
              probability reaches top_p (at least one token)
  temperature the kept logits divided by T; T = 0 means greedy (the first candidate)
  sample      u in [0, 1) from SplitMix64 at counter (seed, step); weights w_i = e^(l_i - l_0)
              over the kept candidates; the token is the first i whose running sum of weights
              exceeds u times the total

SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014, and
its public reference implementation): state += 0x9E3779B97F4A7C15, then the output mix
z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
Here the state for (seed, step) is seed + (step + 1) * 0x9E3779B97F4A7C15 (mod 2^64), i.e. the
(step+1)-th output of the generator seeded with `seed`; u = (z >> 11) * 2^-53.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
WINDOW = 64


def f32(x) -> float:
    """The sampler parameters are f32 values (as the library's parameter block holds them)."""
    return float(np.float32(x))


@dataclass
class SamplerParams:
    repeat_penalty: float = 1.0     # 1 = off
    frequency_penalty: float = 0.0  # 0 = off
    presence_penalty: float = 0.0   # 0 = off
    top_k: int = 40                 # 1 <= top_k
    top_p: float = 1.0              # 1 = off
    temperature: float = 1.0        # 0 = greedy


def splitmix64(seed: int, step: int) -> int:
    """The (step+1)-th SplitMix64 output of the generator seeded with `seed`."""
    z = (seed + (step + 1) * GOLDEN) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def uniform(seed: int, step: int) -> float:
    """u in [0, 1) with 53 random bits."""
    return (splitmix64(seed, step) >> 11) * 2.0 ** -53


def penalize(logits, window, p: SamplerParams) -> np.ndarray:
    """f64 penalized logits; `window` holds the last (at most 64) token ids."""
    out = np.asarray(logits, dtype=np.float32).astype(np.float64)
    window = list(window)[-WINDOW:]
    counts = {}
    for t in window:
        counts[int(t)] = counts.get(int(t), 0) + 1
    for t, c in counts.items():
        v = out[t]
        rp = f32(p.repeat_penalty)
        v = v / rp if v > 0 else v * rp
        v = v - c * f32(p.frequency_penalty) - f32(p.presence_penalty)
        out[t] = v
    return out


def candidates(pen: np.ndarray, k: int) -> np.ndarray:
    """Token ids of the k largest values, largest first, ties by the smaller id."""
    order = np.lexsort((np.arange(pen.size), -pen))  # primary key -value, then the id
    return order[:k].astype(np.int64)


def sample(logits, window, p: SamplerParams, seed: int, step: int) -> int:
    pen = penalize(logits, window, p)
    cand = candidates(pen, min(p.top_k, pen.size))
    lc = pen[cand]
    # top-p on the untempered softmax of the candidates
    if f32(p.top_p) < 1.0:
        w = np.exp(lc - lc[0])
        prob = w / w.sum()
        keep, run = 0, 0.0
        for i in range(lc.size):
            run += prob[i]
            keep = i + 1
            if run >= f32(p.top_p):
                break
        cand, lc = cand[:keep], lc[:keep]
    if f32(p.temperature) == 0.0:
        return int(cand[0])
    lt = lc / f32(p.temperature)
    w = np.exp(lt - lt[0])
    total = 0.0
    for x in w:
        total += x
    target = uniform(seed, step) * total
    run = 0.0
    for i in range(w.size):
        run += w[i]
        if run > target:
            return int(cand[i])
    return int(cand[-1])

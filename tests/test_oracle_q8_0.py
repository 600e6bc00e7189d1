"""Pins of the oracle's Q8_0 quantizer against hand-worked blocks and exact rationals."""
import os

import numpy as np
import pytest

from oracle.q8_0 import dequantize_q8_0, quantize_q8_0
from tests.exact import q8_0_block_exact, rn16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_worked_blocks.txt")


def _parse_pairs(text, conv):
    out = {}
    for tok in text.split():
        i, v = tok.split("=")
        out[int(i)] = conv(v)
    return out


def load_worked_blocks():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.rstrip("\n")
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            cur = {"name": line.split()[1]}
            cases.append(cur)
        elif line.startswith("x:"):
            cur["x"] = _parse_pairs(line[2:], float)
        elif line.startswith("q:"):
            cur["q"] = _parse_pairs(line[2:], int)
        elif line.startswith("d16:"):
            cur["d16"] = int(line[4:].strip(), 16)
    return cases


@pytest.mark.parametrize("case", load_worked_blocks(), ids=lambda c: c["name"])
def test_worked_block(case):
    x = np.zeros(32, dtype=np.float32)
    for i, v in case["x"].items():
        x[i] = np.float32(v)
        assert float(x[i]) == v, "fixture value is not an exact f32"
    q, d = quantize_q8_0(x[None, :])
    want = np.zeros(32, dtype=np.int8)
    for i, v in case["q"].items():
        want[i] = v
    np.testing.assert_array_equal(q[0], want)
    assert int(d.view(np.uint16)[0, 0]) == case["d16"]


def test_random_blocks_match_exact_rationals():
    rng = np.random.default_rng(7)
    blocks = [rng.standard_normal(32).astype(np.float32) * np.float32(s)
              for s in (1.0, 0.02, 3e-3, 1e-5, 40.0)]
    # blocks with outliers and with ties planted on the x*id grid
    b = rng.standard_normal(32).astype(np.float32)
    b[3] = 20 * abs(b).max()
    blocks.append(b)
    t = np.zeros(32, dtype=np.float32)
    t[0] = 127
    t[1:] = (np.arange(31) - 15) + 0.5
    blocks.append(t.astype(np.float32))
    for _ in range(60):
        blocks.append((rng.standard_normal(32) * 10 ** rng.uniform(-6, 3)).astype(np.float32))
    x = np.stack(blocks)
    q, d = quantize_q8_0(x)
    for i, blk in enumerate(blocks):
        codes, d16 = q8_0_block_exact(blk)
        np.testing.assert_array_equal(q[i], np.array(codes, dtype=np.int8), err_msg=f"block {i}")
        assert float(d[i, 0]) == d16, f"block {i}"


def test_fp16_conversion_matches_definition():
    # values straddling fp16 rounding boundaries, including subnormals
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.uniform(0, 1, 2000) * 10 ** rng.uniform(-8, 4, 2000),
        np.array([2 ** -25, 3 * 2 ** -25, 2 ** -24, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 65520.0]),
    ]).astype(np.float32)
    got = vals.astype(np.float16)
    for v, g in zip(vals, got):
        from fractions import Fraction
        assert float(g) == rn16(Fraction(float(v))), v


def test_dequantize_is_scale_times_code():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    q, d = quantize_q8_0(x)
    deq = dequantize_q8_0(q, d)
    for r in range(3):
        for k in range(96):
            assert deq[r, k] == float(d[r, k // 32]) * int(q[r, k])
    # reconstruction error is at most half a step (plus the fp16 rounding of d)
    step = d.astype(np.float64).repeat(32, axis=1)
    assert np.all(np.abs(deq - x) <= 0.5 * step * (1 + 2 ** -10) + np.abs(x) * 2 ** -10)


def test_rejects_ragged_rows():
    with pytest.raises(ValueError):
        quantize_q8_0(np.zeros((2, 33), dtype=np.float32))

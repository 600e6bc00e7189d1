"""Q8_0 block quantization, written out plainly (oracle; test infrastructure only).

Sources.  The walkthrough index ("minfer Inference E2E Walkthrough", master table,
stage 10 "CPU matmul kernels") says every matmul multiplies quantized weights by
activations quantized on the fly to Q8_0.  The pages do not print the block format;
it is taken as the workload defines it: blocks of 32 consecutive values along the
reduction axis, each stored as one fp16 scale d = absmax / 127 and 32 int8 codes,
codes rounded half away from zero.  Readings where that is silent:

* the codes use the f32 scale before it is rounded to fp16: d = RN32(amax / 127),
  id = RN32(1 / d) (0 when d == 0), q = round_half_away(RN32(x * id));
* the stored scale is RN16(d): round-to-nearest-even, subnormals kept;
* dequantized value = f64(fp16 d) * q.

Pins (tests/test_oracle_q8_0.py): hand-worked blocks (amax 127 gives d = 1 so
halves round away: 2.5 -> 3, -0.5 -> -1); the f32 value just below 0.5 -> 0; zero
and one-hot blocks; fp16 tie points; and random blocks against an independent
exact-rational implementation of the same definition.
"""
from __future__ import annotations

import numpy as np

QK = 32  # values per Q8_0 block


def quantize_q8_0(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize f32 rows [..., K] (K % 32 == 0) to (codes int8 [..., K], scales f16 [..., K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = x.shape[-1]
    if k % QK:
        raise ValueError(f"row length {k} is not a multiple of {QK}")
    blocks = x.reshape(*x.shape[:-1], k // QK, QK)
    amax = np.abs(blocks).max(axis=-1)                     # exact in f32
    d = amax / np.float32(127.0)                            # one IEEE f32 division
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = np.float32(1.0) / d[nz]                       # one IEEE f32 division
    v = (blocks * inv[..., None]).astype(np.float64)        # f32 product, widened exactly
    # Round half away from zero.  Done in f64, where |v| + 0.5 is exact for any f32 v
    # (rounding in f32 would turn 0.49999997 + 0.5 into 1.0).
    q = np.sign(v) * np.floor(np.abs(v) + 0.5)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(x.shape), d.astype(np.float16)        # fp16 RNE, subnormals kept


def dequantize_q8_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """f64 values d * q of Q8_0 rows (exact: an 11-bit scale times a 7-bit code)."""
    k = codes.shape[-1]
    q = codes.astype(np.float64).reshape(*codes.shape[:-1], k // QK, QK)
    d = scales.astype(np.float64)[..., None]
    return (q * d).reshape(codes.shape)

"""Oracle: a plain, slow CPU implementation of the Q8_0 prefill forward (numpy, f64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP library and never
receives a value computed by it.

Modules:
  q8_0     Q8_0 quantize / dequantize (bit-exact f32 quantizer, fp16 RNE scales)
  ops      one function per graph node (RMSNorm, Q8_0 matmul, QK-norm, NeoX RoPE,
           KV store, causal GQA attention, SwiGLU, embedding, residual add)
  prefill  the whole forward with the tail-row cut and last-token logits
  sampler  penalties -> top-k -> top-p -> temperature -> seeded sample (SplitMix64)

Parity unpinned: the absolute end-to-end logits of the synthetic models have no
external reference value on the pages; they are pinned only through the op pins
and the forward invariants (replay, causality, tail == full, loop-form brute force).
"""
from . import ops, q8_0, prefill, sampler  # noqa: F401
from .prefill import QuantizedWeights, new_kv_regions, prefill_forward, weights_from_arrays  # noqa: F401
from .q8_0 import dequantize_q8_0, quantize_q8_0  # noqa: F401

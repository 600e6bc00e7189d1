"""Seeded synthetic workloads (shapes, seeds and random draws only)."""
from .configs import (GEMM_SWEEP, HEADLINE, LAYER1, MODEL_CONFIGS, QWEN2_0P5B,
                      QWEN2P5_7B, QWEN3_8B, GemmCase, ModelConfig)
from .generate import (gen_gemm_inputs, gen_normal, gen_tensor, gen_token_ids,
                       iter_tensors, positions_for, stream_seed, tensor_specs)

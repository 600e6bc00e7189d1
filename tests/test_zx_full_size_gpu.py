"""Full-size oracle parity of the 7B- and 8B-shaped prefills (the two largest workloads): last-token
logits and the K and V rows of every layer against the oracle, in the launch configuration the
benchmark times.  The oracle needs tens of TFLOP of f64 work on the host (minutes), so these run
after the other GPU tests and print a line per oracle layer while they work."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_transformer_prefill_amd.model import PrefillModel
from tests.gpu_util import need_gpu, say
from tests.test_forward_gpu import SENTINEL, compare_logits, compare_regions

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", ["qwen2p5_7b_pp2048", "qwen3_8b_chunk3072at1024"])
def test_large_configs_match_oracle(name, capsys):
    """Weights are drawn on the device once for the GPU model and drawn again (the same seeded
    streams) for the oracle, which quantizes them with its own quantizer; the 8B-shaped chunk runs
    after its 1024-token prefix on both sides."""
    with capsys.disabled():   # progress lines reach the log while the oracle runs
        dev = need_gpu()
        cfg = synth.MODEL_CONFIGS[name]
        specs = {n: (shape, kind) for n, shape, kind in synth.tensor_specs(cfg)}
        say(f"\nforward {cfg.name}: loading")
        m = PrefillModel(cfg, synth.iter_tensors(cfg, device=dev), cfg.prefix_tokens + cfg.n_tokens, cfg.n_ctx,
                         device=dev, kv_fill=SENTINEL)
        pre_ids, ids = synth.gen_token_ids(cfg)
        pre_pos, pos = synth.positions_for(cfg)
        torch.cuda.synchronize()
        t0 = time.time()
        if cfg.prefix_tokens:
            m.forward(pre_ids, pre_pos)
        torch.cuda.synchronize()
        t1 = time.time()
        logits = m.forward(ids, pos).cpu().numpy()
        t2 = time.time()
        say(f"  GPU: prefix {t1 - t0:.3f} s, chunk {t2 - t1:.3f} s (first call)")
        gk, gv = m.kv_k.cpu().numpy(), m.kv_v.cpu().numpy()
        del m
        torch.cuda.empty_cache()

        def source(n):
            shape, kind = specs[n]
            return synth.gen_tensor(cfg.seed, n, shape, kind, device=dev).cpu().numpy()

        q8 = [n for n, (shape, kind) in specs.items() if kind == "q8"]
        w = oracle.QuantizedWeights(source, q8, cache=True)
        kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx, fill=SENTINEL)
        t3 = time.time()
        tick = lambda il: say(f"  oracle layer {il} done at {time.time() - t3:.0f} s")
        if cfg.prefix_tokens:
            oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv, progress=tick)
        want = oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv, progress=tick)[0]
        say(f"  oracle: {time.time() - t3:.0f} s")
        compare_logits(logits, want, f"{cfg.name} logits")
        compare_regions(gk, gv, kk, vv, cfg.prefix_tokens + cfg.n_tokens, cfg.name)

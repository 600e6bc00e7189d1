"""Prefill benchmark: one JSON line for the 24-layer 0.5B-shaped model on its 512-token prompt.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]

A step is one mi_prefill_forward over the whole 512-token prompt (all layers, the KV stores,
the last-token lm_head) on seeded synthetic Q8_0 weights resident in HBM.  The dominant kernel
(the fused gate|up matmul with the SwiGLU+Q8_0 epilogue) is timed again on its own, at the same
shape and launch configuration, to report its roofline fraction; the GEMM sweep shapes are timed
the same way.  The oracle (CPU) is timed on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, tera-ops/s
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "quantized_transformer_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def timed_loop(fn, reps: int, torch) -> float:
    """Average milliseconds of fn() over reps launches on the current stream (HIP events)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth
    from quantized_transformer_prefill_amd import binding as B
    from quantized_transformer_prefill_amd.model import PrefillModel

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    B.lib()  # fail loudly if the HIP library is not built
    cfg = synth.HEADLINE
    dev = torch.device("cuda:0")
    t0 = time.time()
    model = PrefillModel(cfg, synth.iter_tensors(cfg, device=dev), cfg.n_tokens, cfg.n_ctx, device=dev)
    torch.cuda.synchronize()
    load_s = time.time() - t0
    _, ids = synth.gen_token_ids(cfg)
    _, pos = synth.positions_for(cfg)

    for _ in range(args.warmup):
        model.forward(ids, pos)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        model.forward(ids, pos)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tok_s = cfg.n_tokens / (ms / 1e3)

    # ---- dominant kernel: fused gate|up matmul + SwiGLU + Q8_0 at the forward's shape
    H, F, M = cfg.hidden, cfg.ffn, cfg.n_tokens
    x = synth.gen_normal(1, "bench.x", (M, H), device=dev)
    xc, xs = B.quantize_q8_0(x)
    gu_codes, gu_scales = model.layer_tensors[0]["w_gate_up"]
    ws_bytes = B.lib().mi_gemm_q8_0_workspace_bytes(M, 2 * F, H)
    wsp = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    reps = 200
    k_ms = timed_loop(lambda: B.gemm_swiglu_q8_0(xc, xs, gu_codes, gu_scales, workspace=wsp), reps, torch)
    ops = 2.0 * M * (2 * F) * H
    achieved = ops / (k_ms / 1e3) / 1e12
    traffic = None
    tf = os.path.join(ROOT, "profiles", "traffic_gemm_swiglu_qwen2_0p5b.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("bytes_per_launch")
    roofline = {"bound": "mfma", "kernel": "k_gemm_q8<EPI_SWIGLU_Q8> (gate|up + SwiGLU + Q8_0)",
                "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS (int8)",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(k_ms, 5), "shape_mnk": [M, 2 * F, H], "launches_timed": reps}

    # ---- the Q8_0 GEMM sweep shapes (quantized activations x Q8_0 weights -> f32)
    sweep = []
    if not args.no_sweep:
        for case in synth.GEMM_SWEEP:
            xw, ww = synth.gen_gemm_inputs(case, device=dev)
            ac, as_ = B.quantize_q8_0(xw)
            wc, wsc = B.quantize_q8_0(ww)
            del xw, ww
            need = B.lib().mi_gemm_q8_0_workspace_bytes(case.m, case.n, case.k)
            gws = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
            out = torch.empty(case.m, case.n, dtype=torch.float32, device=dev)
            wmat = B.q8(wc, wsc)
            import ctypes as C

            def run():
                B.check(B.lib().mi_gemm_q8_0_ws(ac.data_ptr(), as_.data_ptr(), case.m, C.byref(wmat), None, None,
                                                out.data_ptr(), gws.data_ptr(), gws.numel(), 0, B.stream_ptr()))
            g_ms = timed_loop(run, 50, torch)
            tops = 2.0 * case.m * case.n * case.k / (g_ms / 1e3) / 1e12
            sweep.append({"mnk": [case.m, case.k, case.n], "ms": round(g_ms, 4), "tops": round(tops, 1),
                          "int8_peak_frac": round(tops / INT8_PEAK_TOPS, 4)})
            del ac, as_, wc, wsc, gws, out

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, model_tensors=None)

    line = {
        "metric": "prefill tokens/sec (512-tok prompt) + Q8_0 GEMM % of int8 MFMA peak, 1 GPU",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q8_0 int8 MFMA, f64 accumulation, f32 activations",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q8_0, uniform token ids)",
        "config": {"workload": cfg.name, "description": cfg.description, "n_tokens": cfg.n_tokens,
                   "n_ctx": cfg.n_ctx, "parallelism": "single GPU"},
        "roofline": roofline,
        "gemm_sweep": sweep,
        "cpu_baseline": cpu,
        "load_s": round(load_s, 2),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, model_tensors=None):
    """Time the oracle (numpy, f64 GEMMs) on the first layers of the same model and prompt."""
    import threadpoolctl
    import torch

    import oracle
    import synth

    n_layers = 2
    sample = cfg.with_(n_layers=n_layers)
    q8 = [n for n, s, k in synth.tensor_specs(sample) if k == "q8"]
    dev = torch.device("cuda:0")
    arrays = {n: t.cpu().numpy() for n, k, t in synth.iter_tensors(sample, device=dev)}
    w = oracle.weights_from_arrays(arrays, q8)
    for n in q8:
        w[n]  # quantize outside the timed region
    _, ids = synth.gen_token_ids(cfg)
    _, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(sample, cfg.n_ctx)
    threads = sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info() if i.get("internal_api") == "openblas")
    t0 = time.time()
    oracle.prefill_forward(sample, w, ids, pos, cfg.n_ctx, kk, vv)
    t = time.time() - t0
    scaled = t * cfg.n_layers / n_layers  # lm_head counted n_layers/2 times: a conservative rate
    return {"value": round(cfg.n_tokens / scaled, 2), "unit": "tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{cfg.n_tokens}-token prompt through {n_layers} of {cfg.n_layers} layers plus the "
                      f"lm_head ({t:.1f} s), time scaled by {cfg.n_layers}/{n_layers}",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()

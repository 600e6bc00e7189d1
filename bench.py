"""Prefill benchmark: one JSON line for the 24-layer 0.5B-shaped model on its 512-token prompt.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
    python bench.py --counter-run | --write-counters C F W OUT     (per-kernel counter summary)
    python bench.py --write-wave-states DIR OUT                     (wave states of a --counter-run pass)

A step is one forward over the whole 512-token prompt (all layers, the KV stores, the last-token
lm_head) on seeded synthetic Q8_0 weights resident in HBM, launched as a replay of the captured
forward (mi_prefill_graph_launch: host validation, H2D of ids and positions, graph replay); the
eager call (mi_prefill_forward) is timed too and reported as eager_ms_per_step.  The dominant kernel
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
F64_VALU_PEAK_TFLOPS = 78.6  # MI355X fp64 vector: 256 CUs x 2.4 GHz x 128 flop/clk
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = "traffic_gemm_swiglu_qwen2_0p5b.json"
COPY_BYTES = 256 << 20       # the calibration kernel reads and writes this many bytes


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--traffic-run", action="store_true",
                   help="launch only the dominant kernel (20x) and a 256 MiB streaming kernel (5x), for a "
                        "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE pass")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn the two counter passes of --traffic-run into profiles/" + TRAFFIC_FILE)
    p.add_argument("--counter-run", action="store_true",
                   help="launches for the per-kernel counters: two eager forwards, then the calibration kernel")
    p.add_argument("--write-counters", nargs=4, metavar=("COMPUTE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT"),
                   help="turn the three counter passes of --counter-run into a per-kernel summary (OUT)")
    p.add_argument("--k-sweep", action="store_true",
                   help="time the fused gate|up matmul of the workload's shape at K = 128 .. 3584 and fit a fixed "
                        "plus per-stage (128 K values) cost; prints its own JSON line")
    p.add_argument("--write-wave-states", nargs=2, metavar=("DIR", "OUT"),
                   help="turn a --counter-run pass with the wave-state counters into a per-kernel summary (OUT)")
    p.add_argument("--write-kernel-summary", nargs=2, metavar=("TRACE_DIR", "OUT"),
                   help="turn a rocprofv3 --kernel-trace run of this benchmark into a per-forward kernel table "
                        "(OUT); --skip-forwards leaves out the first forwards, --trace-command records the command")
    p.add_argument("--skip-forwards", type=int, default=1)
    p.add_argument("--trace-command", default="")
    p.add_argument("--decode", action="store_true",
                   help="time decode steps (one token per step, mi_decode_step via a captured graph) after "
                        "the workload's prompt instead of the prefill; prints its own JSON line")
    p.add_argument("--slots", type=int, default=0,
                   help="time one call of N independent sequences (mi_prefill_forward_slots) that split the "
                        "workload's prompt evenly, each with its own KV regions; prints its own JSON line")
    p.add_argument("--probes", action="store_true",
                   help="run the rate probes (libmi_probes.so: f64 FMA, int8 MFMA, the matmul's block loop with "
                        "the exact f64 and with an f32 epilogue) and print their rates as one JSON line")
    p.add_argument("--workload", default=None,
                   help="model workload name (default: the 512-token 0.5B-shaped headline); the others "
                        "are reported for context: " + ", ".join(["layer1_896", "qwen2_0p5b_pp512",
                                                                   "qwen2p5_7b_pp2048", "qwen3_8b_chunk3072at1024"]))
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
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_counters:
        import synth
        write_counters(synth.MODEL_CONFIGS[args.workload] if args.workload else synth.HEADLINE, *args.write_counters)
        return
    if args.write_wave_states:
        import synth
        write_wave_states(synth.MODEL_CONFIGS[args.workload] if args.workload else synth.HEADLINE, *args.write_wave_states)
        return
    if args.write_kernel_summary:
        import synth
        write_kernel_summary(synth.MODEL_CONFIGS[args.workload] if args.workload else synth.HEADLINE,
                             *args.write_kernel_summary, args.skip_forwards, args.trace_command)
        return
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
    cfg = synth.MODEL_CONFIGS[args.workload] if args.workload else synth.HEADLINE
    dev = torch.device("cuda:0")
    if args.probes:
        print(json.dumps({"probes": probe_rates(dev)}), flush=True)
        return
    if args.k_sweep:
        print(json.dumps({"k_sweep": k_sweep(cfg, dev)}), flush=True)
        return
    if args.traffic_run:
        traffic_run(cfg, dev)
        return
    if args.counter_run:
        counter_run(cfg, dev)
        return
    t0 = time.time()
    model = PrefillModel(cfg, synth.iter_tensors(cfg, device=dev), cfg.prefix_tokens + cfg.n_tokens, cfg.n_ctx,
                         device=dev)
    torch.cuda.synchronize()
    load_s = time.time() - t0
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    if cfg.prefix_tokens:  # untimed: the KV rows of the earlier positions; each timed chunk call
        model.forward(pre_ids, pre_pos)  # rewrites the same chunk rows with the same values
        torch.cuda.synchronize()  # the calls below run on another stream
    if args.decode:
        decode_bench(args, cfg, model, ids, pos, load_s)
        return
    if args.slots:
        slots_bench(args, cfg, model, ids, load_s)
        return

    # eager calls (mi_prefill_forward), then the same forward captured once and replayed
    # (mi_prefill_graph_launch: validation, H2D of ids and positions, graph replay) -- the timed
    # steps; both on one side stream, events recorded on it
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            model.forward(ids, pos)
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            model.forward(ids, pos)
        e1.record(stream)
        stream.synchronize()
        eager_ms = e0.elapsed_time(e1) / args.steps
        graph = model.graph(cfg.n_tokens)
        kernels_per_forward = graph.nodes()
        for _ in range(args.warmup):
            graph.launch(ids, pos)
        torch.cuda.synchronize()
        step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        e0.record(stream)
        for i in range(args.steps):
            graph.launch(ids, pos)
            step_ev[i].record(stream)  # per-step spread (the mean below spans e0..e1)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        per_step = [e0.elapsed_time(step_ev[0])] + [step_ev[i - 1].elapsed_time(step_ev[i])
                                                     for i in range(1, args.steps)]
        graph.close()
    tok_s = cfg.n_tokens / (ms / 1e3)

    # ---- dominant kernel: fused gate|up matmul + SwiGLU + Q8_0 at the forward's shape
    run_gu, (M, N2, H) = dominant_kernel(cfg, dev, model.layer_tensors[0]["w_gate_up"])
    reps = 200
    k_ms = timed_loop(run_gu, reps, torch)
    ops = 2.0 * M * N2 * H
    achieved = ops / (k_ms / 1e3) / 1e12
    # the exact scale epilogue: 2 f64 FMAs (4 flops) per output per Q8_0 block, on the VALU
    f64_flops = 4.0 * M * N2 * (H // 32)
    f64_achieved = f64_flops / (k_ms / 1e3) / 1e12
    traffic = None
    tf = os.path.join(ROOT, "profiles", TRAFFIC_FILE)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        # counters taken on this kernel's current source and at this very shape only
        if rec.get("kernel_source_hash") == kernel_source_hash() and rec.get("shape_mnk") == [M, N2, H]:
            traffic = rec.get("bytes_per_launch")
    # the ceiling of this kernel's instruction mix: its block loop (1 x 2 wave tile, exact f64
    # epilogue) with operands in registers, measured now on this GPU
    rates = probe_rates(dev, only=("loop_exact_1x2",))
    ceiling = {"what": "the matmul's block loop alone (1 x 2 wave tile, int8 MFMA + exact f64 epilogue, "
                       "operands in registers, no memory traffic)",
               "achieved": rates["loop_exact_1x2"]["rate"], "unit": "TOP/s (int8)",
               "frac": round(rates["loop_exact_1x2"]["rate"] / INT8_PEAK_TOPS, 4)}
    roofline = {"bound": "mfma", "kernel": "k_gemm_q8<EPI_SWIGLU_Q8> (gate|up + SwiGLU + Q8_0)",
                "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "algorithmic_ops_per_launch": ops, "avg_launch_ms": round(k_ms, 5), "shape_mnk": [M, N2, H],
                "launches_timed": reps, "ceiling": ceiling,
                "f64_epilogue": {"bound": "alu", "achieved": round(f64_achieved, 2), "peak": F64_VALU_PEAK_TFLOPS,
                                 "unit": "TFLOP/s (f64 vector)", "frac": round(f64_achieved / F64_VALU_PEAK_TFLOPS, 4),
                                 "flops_per_launch": f64_flops}}

    # ---- the Q8_0 GEMM sweep shapes (quantized activations x Q8_0 weights -> f32)
    sweep = []
    if not args.no_sweep:
        for case in synth.GEMM_SWEEP:
            xw, ww = synth.gen_gemm_inputs(case, device=dev)
            ac, as_ = B.quantize_q8_0(xw)
            wc, wsc = B.quantize_q8_0(ww)
            del ww
            need = B.lib().mi_gemm_q8_0_workspace_bytes(case.m, case.n, case.k)
            gws = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
            out = torch.empty(case.m, case.n, dtype=torch.float32, device=dev)
            wmat = B.q8(wc, wsc)
            import ctypes as C

            def run():
                B.check(B.lib().mi_gemm_q8_0_ws(ac.data_ptr(), as_.data_ptr(), case.m, C.byref(wmat), None, None,
                                                out.data_ptr(), gws.data_ptr(), gws.numel(), 0, B.stream_ptr()))

            def run_pair():  # the f32 activations quantized on the fly, then the matmul
                B.check(B.lib().mi_quantize_q8_0(xw.data_ptr(), case.m, case.k, ac.data_ptr(), as_.data_ptr(),
                                                 B.stream_ptr()))
                run()
            g_ms = timed_loop(run, 50, torch)
            p_ms = timed_loop(run_pair, 50, torch)
            tops = 2.0 * case.m * case.n * case.k / (g_ms / 1e3) / 1e12
            sweep.append({"mnk": [case.m, case.k, case.n], "ms": round(g_ms, 4), "tops": round(tops, 1),
                          "int8_peak_frac": round(tops / INT8_PEAK_TOPS, 4),
                          "quantize_plus_gemm_ms": round(p_ms, 4)})
            del xw, ac, as_, wc, wsc, gws, out

    box = box_probe(dev)  # right after the GPU work, before the GPU idles through the CPU baseline

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg)

    line = {
        "metric": "prefill tokens/sec (512-tok prompt) + Q8_0 GEMM % of int8 MFMA peak, 1 GPU",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q8_0 int8 MFMA, f64 accumulation, f32 activations",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q8_0, uniform token ids)",
        "config": {"workload": cfg.name, "description": cfg.description, "n_tokens": cfg.n_tokens,
                   "n_ctx": cfg.n_ctx, "parallelism": "single GPU"},
        "ms_per_step_median": round(float(np.median(per_step)), 4),
        "ms_per_step_stdev": round(float(np.std(per_step)), 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "kernels_per_forward": kernels_per_forward,
        "roofline": roofline,
        "gemm_sweep": sweep,
        "cpu_baseline": cpu,
        "box_probe": box,
        "load_s": round(load_s, 2),
    }
    print(json.dumps(line), flush=True)


def box_probe(dev):
    """The register-only int8 MFMA probe, run right after the timed region: its share of the peak
    tracks the clock the GPU ran at, which differs by several percent between hosts."""
    r = probe_rates(dev, only=["mfma_i8"])["mfma_i8"]
    return {"mfma_i8_tops": r["rate"], "int8_peak_frac": r["int8_peak_frac"]}


def slots_bench(args, cfg, model, ids, load_s):
    """One call of n independent sequences splitting the prompt evenly (tokens n_tokens / n each,
    positions 0.. in their own regions), eager, HIP events on a side stream."""
    import torch

    n = args.slots
    per = cfg.n_tokens // n
    if n < 1 or per < 1 or n * per != cfg.n_tokens:
        raise SystemExit(f"--slots must divide the prompt length {cfg.n_tokens}")
    sets = [model.own_kv_set()] + [model.new_kv_set() for _ in range(n - 1)]
    slots = [(ids[i * per:(i + 1) * per], np.arange(per, dtype=np.int32), sets[i]) for i in range(n)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            model.forward_slots(slots)
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            model.forward_slots(slots)
        e1.record(stream)
        stream.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
    line = {
        "metric": "multi-slot prefill tokens/sec (n sequences in one call), 1 GPU",
        "value": round(cfg.n_tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q8_0 int8 MFMA, f64 accumulation, f32 activations",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q8_0, uniform token ids)",
        "config": {"workload": f"{cfg.name}_{n}slots", "slots": n, "tokens_per_slot": per, "n_ctx": cfg.n_ctx,
                   "description": f"{n} sequences of {per} tokens at positions 0..{per - 1}, own regions each, of "
                                  + cfg.description, "parallelism": "single GPU"},
        "load_s": round(load_s, 2),
    }
    print(json.dumps(line), flush=True)


def decode_step_bytes(cfg, context: float) -> float:
    """Algorithmic HBM bytes of one decode step: every Q8_0 weight once (codes + fp16 scales), the
    K and V rows of `context` positions per layer, the new K/V rows, norm gains and biases."""
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    nq, nkv = cfg.n_head * cfg.head_dim, cfg.n_head_kv * cfg.head_dim
    q8 = 34.0 / 32.0
    per_layer = ((nq + 2 * nkv) * H + H * nq + 2 * F * H + H * F) * q8
    per_layer += 2 * context * nkv * 4 + 2 * nkv * 4 + 2 * H * 4 + (nq + 2 * nkv) * 4 * cfg.qkv_bias
    return cfg.n_layers * per_layer + V * H * q8 + H * 4


def decode_bench(args, cfg, model, ids, pos, load_s):
    """Decode steps after the prompt: the step (mi_prefill_graph_launch of a graph captured for one
    token: validation, H2D of id and position, replay) at positions after the prompt, on one side
    stream with HIP events; the eager mi_decode_step is timed too."""
    import torch

    from quantized_transformer_prefill_amd import binding as B

    model.forward(ids, pos)  # the prompt's KV rows (untimed)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed + 1000)
    n = args.warmup + args.steps
    toks = rng.integers(0, cfg.vocab, size=2 * n).astype(np.int32)
    # the steps follow the prompt; a prompt that fills the context (the 8B-shaped chunk ends at
    # n_ctx - 1) has its last rows rewritten by the steps instead
    p0 = min(int(pos[-1]) + 1, cfg.n_ctx - 2 * n)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(args.warmup):
            model.decode(int(toks[i]), p0 + i)
        stream.synchronize()
        e0.record(stream)
        for i in range(args.warmup, n):
            model.decode(int(toks[i]), p0 + i)
        e1.record(stream)
        stream.synchronize()
        eager_ms = e0.elapsed_time(e1) / args.steps
        graph = model.graph(1)
        for i in range(n, n + args.warmup):
            graph.launch(toks[i:i + 1], [p0 + i])
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n + args.warmup, 2 * n):
            graph.launch(toks[i:i + 1], [p0 + i])
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        graph.close()
    # the sampler on the last step's logits (penalties over a 64-token window, top-k 40, top-p 0.9,
    # temperature 0.8), timed alone on the default stream
    sp = type("P", (), dict(repeat_penalty=1.1, frequency_penalty=0.0, presence_penalty=0.0, top_k=40, top_p=0.9,
                            temperature=0.8))
    ws = torch.empty(B.lib().mi_sampler_workspace_bytes(), dtype=torch.uint8, device=model.device)
    tok = torch.empty(1, dtype=torch.int32, device=model.device)
    win = toks[:64]
    samp_ms = timed_loop(lambda: B.sample(model.logits, win, sp, 1, 0, workspace=ws, token_out=tok), 50, torch)
    context = p0 + n + args.warmup + args.steps / 2.0  # mean attended positions over the timed steps
    nbytes = decode_step_bytes(cfg, context)
    gbs = nbytes / (ms / 1e3) / 1e9
    box = box_probe(model.device)
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(cfg)
    line = {
        "metric": "decode tokens/sec (one token per step after the prompt), 1 GPU",
        "value": round(1e3 / ms, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q8_0 (sdot4 int8 dot products), f64 accumulation, f32 activations",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q8_0, uniform token ids)",
        "config": {"workload": cfg.name + "_decode", "description": "decode steps after the prompt of " + cfg.description,
                   "prompt_tokens": cfg.n_tokens, "first_position": p0, "n_ctx": cfg.n_ctx,
                   "parallelism": "single GPU"},
        "eager_ms_per_step": round(eager_ms, 4),
        "sampler_ms": round(samp_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "whole decode step (matrix-vector kernels, attention, lm_head)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_step": round(nbytes), "mean_context": context},
        "cpu_baseline": cpu,
        "box_probe": box,
        "load_s": round(load_s, 2),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_decode(cfg, min_seconds: float = 10.0, max_reps: int = 64):
    """The oracle on decode steps of the same model after the same prompt (the prompt's prefill is
    untimed); weights quantized beforehand."""
    import threadpoolctl
    import torch

    import oracle
    import synth

    q8 = [n for n, s, k in synth.tensor_specs(cfg) if k == "q8"]
    dev = torch.device("cuda:0")
    arrays = {n: t.cpu().numpy() for n, k, t in synth.iter_tensors(cfg, device=dev)}
    w = oracle.weights_from_arrays(arrays, q8)
    for n in q8:
        w[n]
        del arrays[n]
    _, ids = synth.gen_token_ids(cfg)
    _, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx)
    oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)
    threads = sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info() if i.get("internal_api") == "openblas")
    rng = np.random.default_rng(cfg.seed + 2000)
    p0 = int(pos[-1]) + 1
    reps, t = 0, 0.0
    while reps < max_reps and (reps == 0 or t < min_seconds) and p0 + reps < cfg.n_ctx:
        tok = np.array([rng.integers(0, cfg.vocab)], np.int32)
        t0 = time.time()
        oracle.prefill_forward(cfg, w, tok, np.array([p0 + reps], np.int32), cfg.n_ctx, kk, vv)
        t += time.time() - t0
        reps += 1
    return {"value": round(reps / t, 2), "unit": "tokens/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{reps} decode steps (one token each, all {cfg.n_layers} layers and the lm_head) after the "
                      f"{cfg.n_tokens}-token prompt ({t:.1f} s of CPU time; prompt prefill and weight "
                      f"quantization untimed)",
            "host_cpus": os.cpu_count(), **host_info()}


PROBES = {  # name: (probe id of mi_probes.h, workgroups, iterations, unit of the work)
    "f64_fma": (0, 2048, 20000, "T FMA/s"),
    "mfma_i8": (1, 2048, 5000, "TOP/s (int8)"),
    "loop_exact_1x2": (2, 3072, 500, "TOP/s (int8)"),
    "loop_exact_4x2": (3, 2048, 200, "TOP/s (int8)"),
    "loop_f32_2x2": (4, 2048, 2000, "TOP/s (int8)"),
}


def probe_rates(dev, only=None):
    """Rates of the probe kernels (libmi_probes.so), each timed over 5 launches with HIP events on
    the stream they run on, after one untimed launch."""
    import ctypes as C

    import torch

    from quantized_transformer_prefill_amd import binding as B

    lib = C.CDLL(os.path.join(ROOT, "quantized_transformer_prefill_amd", "libmi_probes.so"))
    lib.mi_probe_run.restype = C.c_int
    lib.mi_probe_run.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.POINTER(C.c_double), C.c_void_p]
    out = {}
    for name, (pid, wg, iters, unit) in PROBES.items():
        if only and name not in only:
            continue
        buf = torch.empty(wg * 256, dtype=torch.float64, device=dev)
        work = C.c_double()

        def run():
            rc = lib.mi_probe_run(pid, wg, iters, buf.data_ptr(), C.byref(work), B.stream_ptr())
            if rc:
                raise RuntimeError(f"mi_probe_run({name}) failed: {rc}")
        ms = timed_loop(run, 5, torch)
        rate = work.value / (ms / 1e3) / 1e12
        rec = {"rate": round(rate, 2), "unit": unit, "ms_per_launch": round(ms, 4)}
        if unit.startswith("TOP"):
            rec["int8_peak_frac"] = round(rate / INT8_PEAK_TOPS, 4)
        else:
            rec["f64_peak_frac"] = round(2 * rate / F64_VALU_PEAK_TFLOPS, 4)
        out[name] = rec
    return out


def dominant_kernel(cfg, dev, w_gate_up=None):
    """A callable launching the fused gate|up matmul + SwiGLU + Q8_0 of layer 0 on the forward's
    shape (M = prompt tokens, N = 2 x ffn interleaved rows, K = hidden), and that shape."""
    import torch

    import synth
    from quantized_transformer_prefill_amd import binding as B
    from quantized_transformer_prefill_amd.model import interleave_gate_up

    H, F, M = cfg.hidden, cfg.ffn, cfg.n_tokens
    if w_gate_up is None:
        g = B.quantize_q8_0(synth.gen_tensor(cfg.seed, "blk.0.ffn_gate.weight", (F, H), "q8", device=dev))
        u = B.quantize_q8_0(synth.gen_tensor(cfg.seed, "blk.0.ffn_up.weight", (F, H), "q8", device=dev))
        w_gate_up = (interleave_gate_up(g[0], u[0]).contiguous(), interleave_gate_up(g[1], u[1]).contiguous())
    x = synth.gen_normal(1, "bench.x", (M, H), device=dev)
    xc, xs = B.quantize_q8_0(x)
    ws_bytes = B.lib().mi_gemm_q8_0_workspace_bytes(M, 2 * F, H)
    wsp = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    gu_codes, gu_scales = w_gate_up
    return (lambda: B.gemm_swiglu_q8_0(xc, xs, gu_codes, gu_scales, workspace=wsp)), (M, 2 * F, H)


def k_sweep(cfg, dev):
    """The fused gate|up matmul + SwiGLU + Q8_0 at the workload's M and N = 2 x ffn with K = 128 ..
    3584 (1 .. 28 stages of 128), 200 launches each, and the least-squares fit time = fixed + stages
    x per-stage: how much of a launch grows with the reduction and how much does not."""
    import torch

    import synth
    from quantized_transformer_prefill_amd import binding as B
    from quantized_transformer_prefill_amd.model import interleave_gate_up

    M, F = cfg.n_tokens, cfg.ffn
    pts = []
    for K in (128, 256, 512, 896, 1792, 3584):
        g = B.quantize_q8_0(synth.gen_normal(2, f"ks.g{K}", (F, K), std=0.02, device=dev))
        u = B.quantize_q8_0(synth.gen_normal(3, f"ks.u{K}", (F, K), std=0.02, device=dev))
        wc, ws = interleave_gate_up(g[0], u[0]).contiguous(), interleave_gate_up(g[1], u[1]).contiguous()
        xc, xs = B.quantize_q8_0(synth.gen_normal(1, f"ks.x{K}", (M, K), device=dev))
        wsp = torch.empty(max(B.lib().mi_gemm_q8_0_workspace_bytes(M, 2 * F, K), 8), dtype=torch.uint8, device=dev)
        us = 1e3 * timed_loop(lambda: B.gemm_swiglu_q8_0(xc, xs, wc, ws, workspace=wsp), 200, torch)
        pts.append((K // 128, round(us, 3)))
    st = np.array([p[0] for p in pts], float)
    t = np.array([p[1] for p in pts], float)
    per, fixed = np.polyfit(st, t, 1)
    return {"shape_mn": [M, 2 * F], "stages_us": pts, "fixed_us": round(float(fixed), 2),
            "per_stage_us": round(float(per), 3), "command": f"python3 bench.py --workload {cfg.name} --k-sweep"}


def traffic_run(cfg, dev):
    """Launches for the HBM-traffic counters: the dominant kernel 20 times, then a streaming kernel
    that reads and writes COPY_BYTES (torch's elementwise multiply) 5 times, to calibrate the
    counters against a known byte count."""
    import torch

    run, shape = dominant_kernel(cfg, dev)
    for _ in range(20):
        run()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": cfg.name, "shape_mnk": list(shape), "copy_bytes": COPY_BYTES}), flush=True)


COUNTERS_COMPUTE = ["SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_INSTS_VALU_MFMA_MOPS_F64", "SQ_VALU_MFMA_BUSY_CYCLES",
                    "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_FMA_F64", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                    "SQ_LDS_BANK_CONFLICT"]


def counter_run(cfg, dev):
    """Launches for the per-kernel counters: the model is built, the prompt prefilled twice (eager
    mi_prefill_forward), then the streaming calibration kernel of traffic_run."""
    import torch

    import synth
    from quantized_transformer_prefill_amd.model import PrefillModel

    model = PrefillModel(cfg, synth.iter_tensors(cfg, device=dev), cfg.prefix_tokens + cfg.n_tokens, cfg.n_ctx,
                         device=dev)
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    if cfg.prefix_tokens:
        model.forward(pre_ids, pre_pos)
    for _ in range(2):
        model.forward(ids, pos)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": cfg.name, "forwards": 2, "copy_bytes": COPY_BYTES}), flush=True)


def _dispatch_table(d):
    """{dispatch id: (kernel name, grid size, {counter: value summed over the dispatch's rows})} and
    {dispatch id: duration ns} (from the kernel trace of the same run, when present)."""
    import csv
    import glob

    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                did = int(r["Dispatch_Id"])
                name, grid, vals = out.setdefault(did, (r["Kernel_Name"], r.get("Grid_Size", ""), {}))
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out, dur


def _short(name):
    """mi::kernel<template args> of a trace's kernel name."""
    import re

    m = re.search(r"mi::(\w+)(<[^(]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name


def _gemm_args(short):
    """(RG, CG, EPI, split) of a k_gemm_q8 instance name, or None."""
    import re

    m = re.match(r"k_gemm_q8<(\d+), (\d+), (\d+), (true|false)", short or "")
    return (int(m.group(1)), int(m.group(2)), int(m.group(3)), m.group(4) == "true") if m else None


def _classify(short, prev):
    """The forward node a kernel launch is, from its name and the launch before it."""
    ga = _gemm_args(short)
    if ga:
        epi, split = ga[2], ga[3]
        if epi == 2:
            return "qkv"
        if epi == 1:
            return "gate_up"
        pa = _gemm_args(prev)
        if prev and prev.startswith("k_attention"):
            return "wo_split" if split else "wo"
        if pa and pa[2] == 1:
            return "down_split" if split else "down"
        return "gemm_other"
    if short.startswith("k_rmsnorm_quant"):
        pa = _gemm_args(prev)
        return "norm_partials" if pa and pa[3] else "norm"
    if short.startswith("k_attention"):
        return "attention"
    if short.startswith("k_gemv_q8<4, 1, 1>"):
        return "lm_head"
    if short.startswith("k_embed"):
        return "embed"
    return None


def _forward_kernels(cfg):
    """{node: (label, algorithmic int8 ops per launch or 0, algorithmic HBM bytes per launch)} of
    the forward's nodes at the full prompt (the split-K variants write, and the RMSNorm after them
    reads, two f64 partials per output: the library's split at these shapes)."""
    M, H, F = cfg.n_tokens, cfg.hidden, cfg.ffn
    nq, nkv = cfg.n_head * cfg.head_dim, cfg.n_head_kv * cfg.head_dim
    kv_rows = cfg.prefix_tokens + cfg.n_tokens
    q8 = lambda rows, cols: rows * cols * 34 // 32
    return {
        "gate_up": (f"gate|up + SwiGLU + Q8_0 ({M}x{2 * F}x{H})", 2 * M * 2 * F * H, q8(2 * F, H) + q8(M, H) + q8(M, F)),
        "down_split": (f"down, split-K partials ({M}x{H}x{F})", 2 * M * H * F, q8(H, F) + q8(M, F) + 2 * 8 * M * H),
        "down": (f"down + residual ({M}x{H}x{F})", 2 * M * H * F, q8(H, F) + q8(M, F) + 8 * M * H),
        "wo_split": (f"Wo, split-K partials ({M}x{H}x{nq})", 2 * M * H * nq, q8(H, nq) + q8(M, nq) + 2 * 8 * M * H),
        "wo": (f"Wo + residual ({M}x{H}x{nq})", 2 * M * H * nq, q8(H, nq) + q8(M, nq) + 8 * M * H),
        "qkv": (f"Q|K|V (+bias) + [QK norm] + RoPE + KV store ({M}x{nq + 2 * nkv}x{H})", 2 * M * (nq + 2 * nkv) * H,
                q8(nq + 2 * nkv, H) + q8(M, H) + 4 * M * (nq + 2 * nkv)),
        "attention": (f"causal GQA attention + Q8_0 of the output ({M} queries, keys up to {kv_rows})", 0,
                      4 * M * nq + 8 * kv_rows * nkv + q8(M, nq)),
        "norm_partials": (f"RMSNorm + Q8_0 ({M}x{H}) reducing 2 split-K partials", 0,
                          M * H * (4 + 4) + 2 * 8 * M * H + q8(M, H)),
        "norm": (f"RMSNorm + Q8_0 ({M}x{H})", 0, M * H * 4 + q8(M, H)),
        "lm_head": (f"last-row lm_head, final RMSNorm in its prologue ({cfg.vocab}x{H})", 0,
                    q8(cfg.vocab, H) + 4 * cfg.vocab),
        "embed": (f"embedding rows ({M}x{H})", 0, q8(M, H) + 4 * M * H),
    }


def write_kernel_summary(cfg, trace_dir, out_path, skip, command):
    """Per-forward kernel table of a kernel trace of this benchmark: a forward runs from an embedding
    launch to the last-row lm_head; the first `skip` forwards are left out (first call, and the
    untimed prefix of a chunked workload)."""
    import collections
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f, newline="") as fh:
            rows += [r for r in csv.DictReader(fh) if "mi::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    fwds, cur, after = [], None, []
    for r in rows:
        k = _short(r["Kernel_Name"])
        if k == "k_embed":
            cur = []
            fwds.append(cur)
        if cur is not None:
            cur.append((k, int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r))
            if k.startswith("k_gemv_q8<4, 1, 1>"):
                cur = None
        else:
            after.append((k, int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r))
    use = fwds[skip:]
    spans = [(f[-1][2] - f[0][1]) / 1e3 for f in fwds]
    agg = collections.defaultdict(lambda: [0, 0.0])
    info = {}
    for f in use:
        for k, a, b, r in f:
            agg[k][0] += 1
            agg[k][1] += (b - a) / 1e3
            info.setdefault(k, f"{r.get('Grid_Size_X', '?')}x{r.get('Grid_Size_Y', '?')}x{r.get('Grid_Size_Z', '?')} "
                               f"x {r.get('Workgroup_Size_X', '?')}, {r.get('VGPR_Count', '?')}, "
                               f"{r.get('LDS_Block_Size', '?')}")
    n = max(len(use), 1)
    lines = [f"# rocprofv3 kernel summary: {cfg.description} ({cfg.name})", "#",
             "# commands (repository root on the GPU host; rocprofv3 run from /tmp with TMPDIR=/tmp):",
             f"#   {command}" if command else "#   (trace command not recorded)",
             f"#   python3 bench.py --workload {cfg.name} --write-kernel-summary <trace dir> <this file> "
             f"--skip-forwards {skip}",
             "# Durations in microseconds, from the kernel trace (End - Start).  A forward runs from the embedding",
             "# launch to the last-row lm_head.  Grid: the trace's grid size in threads (x, y, z) x workgroup size;",
             "# then VGPRs and LDS bytes as the trace reports them.", "#",
             "# forward span (first kernel start -> lm_head end), us: " + ", ".join(f"{x:.0f}" for x in spans),
             f"# per forward = total over forwards {skip + 1}..{len(fwds)} / {len(use)}", "#",
             f"# {'kernel':58s} {'calls/fwd':>9s} {'us/fwd':>9s} {'avg_us':>8s}  grid x block, VGPRs, LDS bytes"]
    tot = 0.0
    for k, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"{k:60s} {c / n:9.1f} {t / n:9.1f} {t / c:8.2f}  {info[k]}")
        tot += t / n
    lines.append(f"# sum of kernel time per forward: {tot:.1f} us")
    end = fwds[-1][-1][2] if fwds else 0
    after = [x for x in after if x[1] >= end]  # launches after the last forward (the roofline loop)
    if after:
        la = collections.defaultdict(list)
        for k, a, b, r in after:
            la[k].append((b - a) / 1e3)
        for k, v in la.items():
            if len(v) >= 20:
                lines.append(f"# standalone loop after the forwards: {k}, {len(v)} launches, mean {np.mean(v):.2f} us, "
                             f"median {np.median(v):.2f} us")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_counters(cfg, cdir, fdir, wdir, out_path):
    """Per-kernel counter summary of --counter-run: int8 and f64 MFMA work, f64 VALU FMAs, MFMA busy
    share, LDS, and HBM bytes (FETCH_SIZE / WRITE_SIZE scaled on the streaming kernel as in
    write_traffic).  Rates use the kernel-trace durations of the compute pass (kernels serialized
    by the counter collection)."""
    comp, dur = _dispatch_table(cdir)
    fet, _ = _dispatch_table(fdir)
    wri, _ = _dispatch_table(wdir)

    def calib(tab, counter):
        # the calibration multiplies are the run's last five elementwise-multiply launches (model
        # loading launches smaller ones earlier)
        v = [(did, vals[counter]) for did, (n, g, vals) in tab.items()
             if ("MulFunctor" in n or "mul_kernel" in n) and counter in vals]
        v = [x for _, x in sorted(v)[-5:]]
        return COPY_BYTES / (float(np.median(v)) * 1024.0) if v else float("nan")

    ff, fw = calib(fet, "FETCH_SIZE"), calib(wri, "WRITE_SIZE")

    def by_node(tab, node):
        """{grid: [(dispatch, counters)]} of the launches of one forward node (by name and predecessor)."""
        groups = {}
        for did, (n, g, vals) in tab.items():
            prev = _short(tab[did - 1][0]) if did - 1 in tab else None
            if _classify(_short(n), prev) == node:
                groups.setdefault(g, []).append((did, vals))
        return groups

    run = f"python3 bench.py --workload {cfg.name} --counter-run"
    lines = [f"# Per-kernel counters: {cfg.description} ({cfg.name})", "",
             "Commands (repository root on the GPU host; run from /tmp with TMPDIR=/tmp):", "",
             "    rocprofv3 --kernel-trace --pmc " + " ".join(COUNTERS_COMPUTE) +
             " --output-format csv -d out/cnt_compute -o p -- " + run,
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d out/cnt_fetch -o p -- " + run,
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d out/cnt_write -o p -- " + run,
             f"    python3 bench.py --workload {cfg.name} --write-counters out/cnt_compute out/cnt_fetch "
             "out/cnt_write profiles/counters_" + cfg.name + ".md", "",
             f"Byte counters scaled on a streaming kernel of {COPY_BYTES >> 20} MiB read + written: FETCH_SIZE x "
             f"{ff:.3f}, WRITE_SIZE x {fw:.3f}.  Per kernel: the group of launches at the full prompt (the most "
             "launches of that kernel), medians over its launches.  Durations are from the kernel trace of the "
             "counter pass (kernels serialized), so rates are lower bounds of the bench's.  MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (duration x 2.4 GHz x 1024 SIMDs); co-exec = VALU issued while the MFMA "
             "unit was busy, as a share of its busy cycles.  int8 ops count the MFMA's all 32 rows (the odd "
             "rows carry the f64 conversion constant, no data), so they are 2x the algorithmic 2MNK.", "",
             "| kernel | launches | us | int8 MFMA ops (vs 2MNK) | int8 TOP/s (% of 5000) | f64 MFMA TFLOP/s | "
             "f64 VALU FMA TFLOP/s (% of 78.6) | MFMA busy | co-exec | LDS bank conflicts / LDS instr | "
             "HBM MB (vs algorithmic) | HBM GB/s (% of 8000) |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    med = lambda xs: float(np.median(xs)) if xs else float("nan")
    for node, (label, ops_alg, bytes_alg) in _forward_kernels(cfg).items():
        label = label.replace("|", "\\|")
        groups = by_node(comp, node)
        if not groups:
            continue
        g, disp = max(groups.items(), key=lambda kv: len(kv[1]))
        ids = [d for d, _ in disp]
        dns = med([dur[d] for d in ids if d in dur])
        cv = lambda c: med([v.get(c, float("nan")) for _, v in disp])
        i8 = cv("SQ_INSTS_VALU_MFMA_MOPS_I8") * 512
        f64m = cv("SQ_INSTS_VALU_MFMA_MOPS_F64") * 512
        fma64 = cv("SQ_INSTS_VALU_FMA_F64") * 64 * 2
        busy = cv("SQ_VALU_MFMA_BUSY_CYCLES")
        coex = cv("SQ_VALU_MFMA_COEXEC_CYCLES")
        ldsc = cv("SQ_LDS_BANK_CONFLICT") / max(cv("SQ_INSTS_LDS"), 1.0)
        fg = by_node(fet, node).get(g, [])
        wg = by_node(wri, node).get(g, [])
        hbm = (med([v["FETCH_SIZE"] for _, v in fg]) * 1024 * ff if fg else float("nan")) + \
              (med([v["WRITE_SIZE"] for _, v in wg]) * 1024 * fw if wg else float("nan"))
        s_ = dns * 1e-9
        r8 = i8 / s_ / 1e12
        lines.append(
            f"| {label} | {len(disp)} | {dns / 1e3:.1f} | {i8 / 1e9:.2f} G"
            + (f" ({i8 / ops_alg:.2f}x)" if ops_alg else "") + f" | {r8:.0f} ({100 * r8 / INT8_PEAK_TOPS:.1f}%) | "
            f"{f64m / s_ / 1e12:.1f} | {fma64 / s_ / 1e12:.1f} ({100 * fma64 / s_ / 1e12 / F64_VALU_PEAK_TFLOPS:.0f}%) | "
            f"{100 * busy / (s_ * 2.4e9 * 1024):.0f}% | {100 * coex / busy if busy else 0:.0f}% | {ldsc:.3f} | "
            f"{hbm / 1e6:.2f} ({hbm / bytes_alg:.2f}x) | {hbm / s_ / 1e9:.0f} ({100 * hbm / s_ / 1e9 / HBM_PEAK_GBS:.0f}%) |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS_WAVE = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                 "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS"]


def write_wave_states(cfg, d, out_path):
    """Where a wave's life goes, per forward node, from one --counter-run pass with COUNTERS_WAVE:
    waiting on a counter or barrier (SQ_WAIT_ANY), ready but not issued (SQ_WAIT_INST_ANY), issuing
    (SQ_ACTIVE_INST_ANY), each as a share of SQ_WAVE_CYCLES; and the VALU, scalar and LDS issue
    cycles per wave (the counters count in units of 4 cycles)."""
    tab, _ = _dispatch_table(d)

    def by_node(node):
        groups = {}
        for did, (n, g, vals) in tab.items():
            prev = _short(tab[did - 1][0]) if did - 1 in tab else None
            if _classify(_short(n), prev) == node:
                groups.setdefault(g, []).append(vals)
        return groups

    run = f"python3 bench.py --workload {cfg.name} --counter-run"
    lines = [f"# Wave states per kernel: {cfg.description} ({cfg.name})", "",
             "Commands (repository root on the GPU host; run from /tmp with TMPDIR=/tmp):", "",
             "    rocprofv3 --pmc " + " ".join(COUNTERS_WAVE) + " --output-format csv -d out/cnt_wave -o p -- " + run,
             f"    python3 bench.py --workload {cfg.name} --write-wave-states out/cnt_wave "
             f"profiles/wave_states_{cfg.name}.md", "",
             "Per kernel: the group of launches at the full prompt, medians over its launches.  Shares of the "
             "summed wave cycles (SQ_WAVE_CYCLES): waiting on a counter or the barrier (SQ_WAIT_ANY), ready but "
             "not issued (SQ_WAIT_INST_ANY), issuing (SQ_ACTIVE_INST_ANY).  Issue cycles per wave: "
             "SQ_ACTIVE_INST_VALU, _SCA, _LDS x 4 / SQ_WAVES (the counters count in units of 4 cycles).", "",
             "| kernel | launches | waves | cycles per wave | waiting | ready, not issued | issuing | "
             "VALU cycles per wave | scalar cycles per wave | LDS cycles per wave |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    med = lambda xs: float(np.median(xs)) if xs else float("nan")
    for node, (label, _, _) in _forward_kernels(cfg).items():
        groups = by_node(node)
        if not groups:
            continue
        _, disp = max(groups.items(), key=lambda kv: len(kv[1]))
        cv = lambda c: med([v.get(c, float("nan")) for v in disp])
        waves, wc = cv("SQ_WAVES"), cv("SQ_WAVE_CYCLES")
        share = lambda c: 100.0 * cv(c) / wc if wc else float("nan")
        per = lambda c: 4.0 * cv(c) / waves if waves else float("nan")
        lines.append(f"| {label.replace('|', chr(92) + '|')} | {len(disp)} | {waves:.0f} | {4.0 * wc / waves:.0f} | "
                     f"{share('SQ_WAIT_ANY'):.0f}% | {share('SQ_WAIT_INST_ANY'):.0f}% | {share('SQ_ACTIVE_INST_ANY'):.0f}% | "
                     f"{per('SQ_ACTIVE_INST_VALU'):.0f} | {per('SQ_ACTIVE_INST_SCA'):.0f} | "
                     f"{per('SQ_ACTIVE_INST_LDS'):.0f} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(d, counter):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(fetch_dir, write_dir, shape=(512, 9728, 896)):
    """HBM bytes per launch of the dominant kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by the factor that maps the same counter onto the known bytes of the streaming kernel."""
    out = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        gemm = [v for n, v in rows if "k_gemm_q8" in n]
        copy = [v for n, v in rows if "MulFunctor" in n or "mul_kernel" in n]
        if not gemm or not copy:
            raise SystemExit(f"{counter}: gemm dispatches {len(gemm)}, calibration dispatches {len(copy)}")
        copy_kib = float(np.median(copy))
        factor = COPY_BYTES / (copy_kib * 1024.0)
        out[key] = {"counter": counter, "kernel_kib_median": float(np.median(gemm)), "dispatches": len(gemm),
                    "calibration_kib_median": copy_kib, "calibration_bytes": COPY_BYTES, "factor": factor,
                    "bytes_per_launch": float(np.median(gemm)) * 1024.0 * factor}
    rec = {"kernel": "k_gemm_q8<EPI_SWIGLU_Q8> (gate|up + SwiGLU + Q8_0), %d x %d x %d" % tuple(shape),
           "shape_mnk": list(shape),
           "kernel_source_hash": kernel_source_hash(),
           "bytes_per_launch": round(out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]),
           "fetch": out["fetch"], "write": out["write"],
           "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d out/pmc_fetch -o p -- "
                        "python3 bench.py --traffic-run",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d out/pmc_write -o p -- "
                        "python3 bench.py --traffic-run",
                        "python3 bench.py --write-traffic out/pmc_fetch out/pmc_write"]}
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def cpu_baseline(cfg, min_seconds: float = 10.0, max_reps: int = 8):
    """Time the oracle (numpy, f64 GEMMs) on whole forwards of the same model and prompt.

    The sample is the full prefill call (every layer, the KV stores, the last-token lm_head),
    repeated until min_seconds of CPU time have passed or max_reps calls ran; weight
    quantization happens before the timed region, as the GPU side loads its weights untimed.
    """
    import threadpoolctl
    import torch

    import oracle
    import synth

    q8 = [n for n, s, k in synth.tensor_specs(cfg) if k == "q8"]
    dev = torch.device("cuda:0")
    arrays = {n: t.cpu().numpy() for n, k, t in synth.iter_tensors(cfg, device=dev)}
    w = oracle.weights_from_arrays(arrays, q8)
    for n in q8:
        w[n]  # quantize outside the timed region
        del arrays[n]  # the f32 originals of quantized weights are no longer read
    pre_ids, ids = synth.gen_token_ids(cfg)
    pre_pos, pos = synth.positions_for(cfg)
    kk, vv = oracle.new_kv_regions(cfg, cfg.n_ctx)
    if cfg.prefix_tokens:
        oracle.prefill_forward(cfg, w, pre_ids, pre_pos, cfg.n_ctx, kk, vv)
    threads = sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info() if i.get("internal_api") == "openblas")
    reps, t = 0, 0.0
    while reps < max_reps and (reps == 0 or t < min_seconds):
        t0 = time.time()
        oracle.prefill_forward(cfg, w, ids, pos, cfg.n_ctx, kk, vv)
        t += time.time() - t0
        reps += 1
    return {"value": round(reps * cfg.n_tokens / t, 2), "unit": "tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{reps} whole prefill call(s) of the {cfg.n_tokens}-token prompt through all {cfg.n_layers} "
                      f"layers and the lm_head ({t:.1f} s of CPU time; weights quantized beforehand)",
            "host_cpus": os.cpu_count(), **host_info()}


def host_info():
    """The host CPU model and numpy's BLAS, recorded beside the oracle's timing."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        info = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{info.get('name')} {info.get('version')}"
    except Exception:  # numpy builds without the dict form
        pass
    return {"cpu_model": model, "blas": blas}


if __name__ == "__main__":
    main()

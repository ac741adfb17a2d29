"""Benchmark: batched prefill of the Llama-3.2-3B-shaped 28-layer dense stack
at pp512 (512 new tokens, empty cache) on one MI355X, through the C ABI.

A step is one ddl_prefill_dense_stack call over the whole 28-layer run with
weights, hidden rows and outputs resident in HBM.  Prints one JSON line:
tokens/s, the stack's fraction of dense fp16/bf16 MFMA peak, the roofline of
the dominant kernel (the gate/up projection + SwiGLU GEMM, timed per launch
with HIP events in a second pass of the same steps) and the CPU oracle timed
on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s, Llama-3.2-3B-shape 28-layer stack pp512; % bf16 MFMA peak"
PEAK_MFMA_TFLOPS = 2516.6      # dense fp16 = bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(cfg):
    """GEMM flops plus the unmasked causal attention triangle, per call."""
    d, f = cfg.d_model, cfg.d_ff
    qw, kw = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    params = d * (qw * (2 if cfg.gated else 1) + 2 * kw) + d * qw + 3 * d * f
    gemm = 2 * cfg.batch * params
    causal = sum(cfg.start_pos + b + 1 for b in range(cfg.batch))
    attn = 4 * cfg.head_dim * cfg.n_heads * causal
    return (gemm + attn) * cfg.n_layers, 2 * cfg.batch * d * 2 * f


def cpu_baseline(cfg, n_sample_layers=2):
    """The oracle (fp64 numpy) on the first layers of the same workload."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    sub = cfg.replace(n_layers=n_sample_layers)
    inp = synth.stack_inputs(sub)
    layers = [{n: synth.values(a) for n, a in w.items()} for w in inp.layers]
    t0 = time.perf_counter()
    oracle.prefill_dense_stack(inp.hidden, layers, sub, sub.start_pos, inp.prefix_k, inp.prefix_v)
    dt = time.perf_counter() - t0
    per_step = dt * cfg.n_layers / n_sample_layers
    return {"value": cfg.batch / per_step, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_sample_layers} of {cfg.n_layers} layers at pp{cfg.batch} "
                      f"(fp64 numpy oracle, {dt:.1f}s), scaled x{cfg.n_layers / n_sample_layers:g}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding "
                                   "is a design (DESIGN.md), not a launched path",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import dense_decoder_layer_amd as ddl
    import synth
    from dense_decoder_layer_amd.workloads import DeviceStack

    cfg = synth.STACK_CONFIGS["llama3b_pp512"]
    torch.cuda.set_device(0)
    t0 = time.time()
    ctx = ddl.ddl_ctx_create()
    layers_iter = (synth.layer_weights(cfg, l) for l in range(cfg.n_layers))
    stack = DeviceStack(ctx, cfg, layers_iter)
    bufs = stack.buffers(cfg.batch, cfg.start_pos)
    hidden = torch.from_numpy(synth.hidden_rows(cfg)).cuda()
    torch.cuda.synchronize()
    log(f"packed {cfg.n_layers} layers in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        assert stack.run(hidden, 0, None, None, bufs) == cfg.n_layers, ddl.ddl_last_error()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        stack.run(hidden, 0, None, None, bufs)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step")

    # second pass of the same steps: HIP events around every gate/up GEMM launch
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_GEMM_GATE_UP, args.steps * cfg.n_layers)
    for _ in range(args.steps):
        stack.run(hidden, 0, None, None, bufs)
    torch.cuda.synchronize()
    durs = ddl.ddl_probe_read(ctx, args.steps * cfg.n_layers)
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_GEMM_GATE_UP, 0)
    gu_ms = sum(durs) / len(durs)

    flops, gu_flops = algorithmic_flops(cfg)
    tok_s = cfg.batch / (ms / 1e3)
    achieved = gu_flops / (gu_ms / 1e3) / 1e12
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama3b_pp512: 28 dense layers, hidden 3072, 24 q / 8 KV heads "
                               "x 128, SwiGLU 8192, 512 new tokens, start_pos 0, bf16-valued "
                               "weights, fp32 activations", "batch": cfg.batch,
                   "start_pos": cfg.start_pos, "layers": cfg.n_layers},
        "mfma_peak_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "roofline": {"kernel": "gemm gate/up + SwiGLU (512 x 16384 x 3072)", "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "avg_launch_us": round(gu_ms * 1e3, 2), "launches": len(durs),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

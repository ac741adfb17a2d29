"""Benchmark: batched prefill of the Llama-3.2-3B-shaped 28-layer dense stack
at pp512 (512 new tokens, empty cache) on one MI355X, through the C ABI.

A step is one ddl_prefill_dense_stack call over the whole 28-layer run with
weights, hidden rows and outputs resident in HBM.  Prints one JSON line:
tokens/s, the stack's fraction of dense fp16/bf16 MFMA peak, the roofline of
the dominant kernel (the gate/up projection + SwiGLU GEMM, timed per launch
with HIP events in a second pass of the same steps), the single-token decode
layer at 32768 cached rows (ms per layer, decode attention as a fraction of
HBM bandwidth and of a plain device copy's rate), the other prefill
workloads as secondary lines (the 3B stack over a 1536-row cached prefix,
the 8B-shaped stack with biases and QK norms at pp4096) and the CPU oracle
timed on a bounded sample of each workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
                    [--no-decode] [--no-secondary] [--copy-calibration]
                    [--library-gemms]

--copy-calibration adds three plain 1 GiB device-to-device copies at the end,
the reference a hardware-counter run scales FETCH_SIZE / WRITE_SIZE by.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s, Llama-3.2-3B-shape 28-layer stack pp512; % bf16 MFMA peak"
PEAK_MFMA_TFLOPS = 2516.6      # dense fp16 = bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
ATTN_FORMS = {"auto": 0, "one-head": 1, "shared": 2}     # ddl.h DDL_ATTN_*


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


def oracle_cores():
    """The threads the oracle actually runs on: its matrix products use the
    BLAS pool (OMP_NUM_THREADS, the host's CPU share for one GPU); its
    elementwise steps run on one thread."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(cfg, budget_s=12.0, max_layers=None):
    """The oracle (fp64 numpy) layer by layer over the same workload (with
    the layer's cached prefix rows when there are any) until about
    ``budget_s`` seconds of oracle time, ``max_layers`` layers or the whole
    stack have run; drawing the inputs is not timed.  Scaled to the whole
    stack."""
    import oracle
    import synth
    cores = oracle_cores()
    x = synth.hidden_rows(cfg)
    spent, done = 0.0, 0
    limit = cfg.n_layers if max_layers is None else min(max_layers, cfg.n_layers)
    while done < limit and spent < budget_s:
        w = {n: synth.values(a) for n, a in synth.layer_weights(cfg, done).items()}
        pk, pv = synth.prefix_rows(cfg, done) if cfg.start_pos > 0 else (None, None)
        t0 = time.perf_counter()
        x, _, _ = oracle.dense_layer(x, w, cfg, cfg.start_pos, pk, pv)
        spent += time.perf_counter() - t0
        done += 1
    per_step = spent * cfg.n_layers / done
    return {"value": round(cfg.batch / per_step, 2), "unit": "tok/s", "cores": cores,
            "host_nproc": os.cpu_count(), "kind": "oracle",
            "sample": f"first {done} of {cfg.n_layers} layers at pp{cfg.batch}"
                      + (f" over a {cfg.start_pos}-row prefix" if cfg.start_pos else "")
                      + f" (fp64 numpy oracle, {spent:.1f}s), scaled x{cfg.n_layers / done:g}"}


def gate_up_traffic():
    """HBM bytes per gate/up launch from the committed hardware-counter
    summary, or None when the GEMM source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_llama3b_pp512_pmc.md")
    src = os.path.join(ROOT, "dense_decoder_layer_amd", "csrc", "gemm.hip")
    try:
        text = open(path).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    want = re.search(r"gemm\.hip sha256: ([0-9a-f]{64})", text)
    val = re.search(r"traffic bytes per launch: (\d+)", text)
    if not want or not val or want.group(1) != digest:
        return None
    return int(val.group(1))


def decode_bench(ddl, ctx, reps=40):
    """ddl_attn_layer at 32768 cached rows, gated, softcap 50 (one token).
    Two mirrors alternate so the 268 MB of K/V rows a call reads cannot sit
    in the 256 MB last-level cache; each call appends its row, as a decode
    loop does."""
    import numpy as np
    import torch
    import synth
    from dense_decoder_layer_amd.workloads import desc_for
    cfg = synth.DECODE_CONFIG
    inp = synth.decode_inputs(cfg)
    layer = ddl.pack_layer_from_host(ctx, desc_for(cfg.stack_view()), inp["weights"])
    cap = ddl.ddl_mirror_plan_capacity(cfg.rows, cfg.rows + 14 * reps + 32)   # every call appends a row
    mirrors, bufs = [], []
    k = torch.from_numpy(inp["cache_k"]).cuda()
    v = torch.from_numpy(inp["cache_v"]).cuda()
    for _ in range(2):
        buf = torch.empty(ddl.ddl_mirror_bytes(cfg.n_kv_heads, cfg.head_dim, cap),
                          dtype=torch.uint8, device="cuda")
        m = ddl.ddl_mirror_init(buf, cfg.n_kv_heads, cfg.head_dim, cap)
        assert ddl.ddl_mirror_upload(m, k, v, cfg.rows) == 1
        mirrors.append(m)
        bufs.append(buf)
    del k, v
    ws = torch.empty(ddl.ddl_attn_workspace_bytes(layer, cap), dtype=torch.uint8, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, kn, vn, gate, res = (t(inp[n]) for n in ("q", "k", "v", "gate", "residual"))
    out = torch.empty(cfg.d_model, dtype=torch.float32, device="cuda")

    def call(i):
        m = mirrors[i % 2]
        rows = ddl.ddl_mirror_seq_len(m)
        rc = ddl.ddl_attn_layer(ctx, m, rows, q, kn, vn, gate,
                                cfg.n_heads, cfg.softcap, layer, res, out, ws)
        assert rc == 1, ddl.ddl_last_error()
        return rows + 1                 # rows attended: the cached ones and this token's

    for i in range(4):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    start.record(stream)
    for i in range(reps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    layer_ms = start.elapsed_time(end) / reps
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_DECODE_ATTN, reps)
    attended = sum(call(i) for i in range(reps))
    torch.cuda.synchronize()
    durs = ddl.ddl_probe_read(ctx, reps)
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_DECODE_ATTN, 0)
    attn_ms = sum(durs) / len(durs)
    tail = {}
    for name, kind in (("gemv_wo", ddl.DDL_K_GEMV_WO), ("gemv_gate_up", ddl.DDL_K_GEMV_GATE_UP),
                       ("gemv_down", ddl.DDL_K_GEMV_DOWN)):
        ddl.ddl_probe_enable(ctx, kind, reps)
        for i in range(reps):
            call(i)
        torch.cuda.synchronize()
        d = ddl.ddl_probe_read(ctx, reps)
        ddl.ddl_probe_enable(ctx, kind, 0)
        tail[name + "_us"] = round(sum(d) / len(d) * 1e3, 2)
    # the whole layer with its head on the device (ddl_decode_layer): RMS norm,
    # stacked q/k/v/gate GEMV, bias/QK-norm/RoPE, then the same attention and tail
    hid = t(inp["residual"])
    k_row = torch.empty(cfg.kv_width, dtype=torch.float32, device="cuda")
    v_row = torch.empty_like(k_row)

    def dcall(i):
        m = mirrors[i % 2]
        rc = ddl.ddl_decode_layer(ctx, m, ddl.ddl_mirror_seq_len(m), hid, layer, out, k_row, v_row,
                                  ws)
        assert rc == 1, ddl.ddl_last_error()

    for i in range(4):
        dcall(i)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        dcall(i)
    end.record(stream)
    torch.cuda.synchronize()
    full_ms = start.elapsed_time(end) / reps
    for name, kind in (("gemv_qkv", ddl.DDL_K_GEMV_QKV), ("head", ddl.DDL_K_DECODE_HEAD)):
        ddl.ddl_probe_enable(ctx, kind, reps)
        for i in range(reps):
            dcall(i)
        torch.cuda.synchronize()
        d = ddl.ddl_probe_read(ctx, reps)
        ddl.ddl_probe_enable(ctx, kind, 0)
        tail[name + "_us"] = round(sum(d) / len(d) * 1e3, 2)
    # the same step captured once per mirror as a HIP graph and replayed
    graphs = [ddl.ddl_decode_graph_create(ctx, m, layer, hid, out, k_row, v_row, w)
              for m, w in zip(mirrors, (ws, torch.empty_like(ws)))]

    def gcall(i):
        m = mirrors[i % 2]
        rc = ddl.ddl_decode_graph_launch(ctx, graphs[i % 2], ddl.ddl_mirror_seq_len(m))
        assert rc == 1, ddl.ddl_last_error()

    for i in range(4):
        gcall(i)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        gcall(i)
    end.record(stream)
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / reps
    # one token at a time, the host waiting for each (a decode loop that
    # samples between tokens): the submissions of a step are on the path
    sync = {}
    for name, fn in (("decode_layer_sync_ms", dcall), ("decode_graph_sync_ms", gcall)):
        t0 = time.perf_counter()
        for i in range(reps):
            fn(i)
            torch.cuda.synchronize()
        sync[name] = round((time.perf_counter() - t0) / reps * 1e3, 4)
    del graphs
    # the practical HBM roof: a plain 1 GiB device-to-device copy, bytes read
    # plus bytes written over its time, best of 5
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = []
    for _ in range(5):
        start.record(stream)
        dst.copy_(src)
        end.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(start.elapsed_time(end))
    copy_gbs = 2 * src.nbytes / (min(copy_ms) / 1e3) / 1e9
    del src, dst
    attn_bytes = attended * cfg.kv_width * 4 * 2 // reps     # fp32 K and V rows read per call
    # the tail's fp16 weights: wo, gate and up, down
    tail_bytes = 2 * (cfg.d_model * cfg.n_heads * cfg.head_dim + 3 * cfg.d_model * cfg.d_ff)
    return {"config": f"{cfg.name}: {cfg.rows} cached rows, {cfg.n_heads} q / {cfg.n_kv_heads} "
                      f"KV heads x {cfg.head_dim}, softcap {cfg.softcap:g}, sigmoid gate, "
                      f"wo + RMSNorm + SwiGLU {cfg.d_ff} tail, hidden {cfg.d_model}",
            "ms_per_layer": round(layer_ms, 4),
            "decode_layer_ms": round(full_ms, 4),   # ddl_decode_layer: head on the device too
            "decode_graph_ms": round(graph_ms, 4),  # the same step replayed as one HIP graph
            **sync,
            "attn_us": round(attn_ms * 1e3, 2),
            "attn_bytes": attn_bytes,
            "attn_hbm_gbs": round(attn_bytes / (attn_ms / 1e3) / 1e9, 1),
            "attn_hbm_frac": round(attn_bytes / (attn_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "copy_gbs": round(copy_gbs, 1),                # a plain device copy on the same box
            "attn_frac_of_copy": round(attn_bytes / (attn_ms / 1e3) / 1e9 / copy_gbs, 4),
            # ddl_attn_layer's HBM bytes (K/V rows + tail weights) over its time
            "layer_hbm_gbs": round((attn_bytes + tail_bytes) / (layer_ms / 1e3) / 1e9, 1),
            "tail": tail}


def cpu_baseline_decode(reps=3):
    """The oracle's attention layer (fp64 numpy) at the decode workload, 32768
    cached rows, one token per call; drawing and converting the inputs is not
    timed."""
    import oracle
    import synth
    cfg = synth.DECODE_CONFIG
    inp = synth.decode_inputs(cfg)
    w = {n: synth.values(a) for n, a in inp["weights"].items()}
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attn_layer(inp["q"], inp["k"], inp["v"], inp["gate"], inp["cache_k"],
                          inp["cache_v"], cfg.rows, w, cfg, inp["residual"])
    per = (time.perf_counter() - t0) / reps
    return {"ms_per_layer": round(per * 1e3, 2), "cores": oracle_cores(), "kind": "oracle",
            "sample": f"{reps} tokens at {cfg.rows} cached rows (fp64 numpy oracle)"}


def timed_steps(step, steps):
    """Runs `step` `steps` times back to back on the current stream, with an
    event between consecutive steps (no synchronisation inside the timed
    region).  Returns (mean, median, min) ms per step; the mean is the
    whole span over the step count."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, statistics.median(per), min(per)


def _time_stack(stack, hidden, start_pos, pk, pv, bufs, warmup, steps):
    import torch
    for _ in range(warmup):
        assert stack.run(hidden, start_pos, pk, pv, bufs) == len(stack.layers)
    torch.cuda.synchronize()
    return timed_steps(lambda: stack.run(hidden, start_pos, pk, pv, bufs), steps)


def _line(cfg, times, steps, note):
    flops, _ = algorithmic_flops(cfg)
    ms, med, mn = times
    return {"workload": f"{cfg.name}: {cfg.n_layers} layers, hidden {cfg.d_model}, "
                        f"{cfg.n_heads} q / {cfg.n_kv_heads} KV heads x {cfg.head_dim}, "
                        f"FFN {cfg.d_ff}, {cfg.batch} new tokens, start_pos {cfg.start_pos}" + note,
            "tok_s": round(cfg.batch / (ms / 1e3), 1), "ms_per_step": round(ms, 3),
            "ms_median": round(med, 3), "ms_min": round(mn, 3), "steps": steps,
            "algorithmic_tflop_per_step": round(flops / 1e12, 3),
            "mfma_peak_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4)}


def secondary_bench(ddl, ctx, stack3b, hidden3b, args, which=("prefix1536", "pp4096")):
    """The other prefill workloads, each a whole stack per step with inputs
    resident in HBM: the 3B stack over a 1536-row cached prefix per layer
    (the same seeded weights as the headline, so the packed stack is reused),
    and the 8B-shaped stack with q/k/v biases and QK norms at pp4096."""
    import torch
    import synth
    from dense_decoder_layer_amd.workloads import DeviceStack
    out = []
    if "prefix1536" in which:
        cfg = synth.STACK_CONFIGS["llama3b_prefix1536"]
        pk, pv = [], []
        for l in range(cfg.n_layers):
            k, v = synth.prefix_rows(cfg, l)
            pk.append(torch.from_numpy(k).cuda())
            pv.append(torch.from_numpy(v).cuda())
        bufs = stack3b.buffers(cfg.batch, cfg.start_pos)
        steps = max(3, min(args.steps, 10))
        times = _time_stack(stack3b, hidden3b, cfg.start_pos, pk, pv, bufs, 2, steps)
        log(f"3B over a 1536-row prefix: {times[0]:.3f} ms/step")
        out.append(_line(cfg, times, steps, "; prefix K/V rows fp32 resident per layer"))
        del pk, pv, bufs
    if "pp4096" in which:
        cfg = synth.STACK_CONFIGS["llama8b_pp4096_extras"]
        t0 = time.time()
        stack = DeviceStack(ctx, cfg, (synth.layer_weights(cfg, l) for l in range(cfg.n_layers)))
        hidden = torch.from_numpy(synth.hidden_rows(cfg)).cuda()
        bufs = stack.buffers(cfg.batch, 0)
        log(f"packed the 8B stack in {time.time() - t0:.1f}s")
        times = _time_stack(stack, hidden, 0, None, None, bufs, 1, 3)
        log(f"8B pp4096: {times[0]:.3f} ms/step")
        out.append(_line(cfg, times, 3, "; q/k/v biases and per-head QK RMSNorm"))
        del stack, bufs, hidden
    torch.cuda.empty_cache()
    return out


def secondary_only(which, args):
    """One secondary workload alone (for a per-workload profile): prints its
    line, not the headline's."""
    import torch
    import dense_decoder_layer_amd as ddl
    import synth
    from dense_decoder_layer_amd.workloads import DeviceStack
    torch.cuda.set_device(0)
    ctx = ddl.ddl_ctx_create(attn_form=ATTN_FORMS[args.attn_form])
    stack = hidden = None
    if which == "prefix1536":
        cfg = synth.STACK_CONFIGS["llama3b_pp512"]
        stack = DeviceStack(ctx, cfg, (synth.layer_weights(cfg, l) for l in range(cfg.n_layers)))
        hidden = torch.from_numpy(synth.hidden_rows(cfg)).cuda()
    print(json.dumps({"secondary": secondary_bench(ddl, ctx, stack, hidden, args, (which,))}),
          flush=True)


def library_gemms(args):
    """The four projection shapes of the 3B pp512 layer and of the 8B layer at
    4096 tokens through torch's GEMMs
    (the platform's GEMM library, fp16 in, fp16 out), the weight stored K x N
    (torch.matmul) and N x K (torch.nn.functional.linear), each weight
    rotated over four copies so that, as in the stack, it comes from HBM: a
    yardstick for the GEMM kernels' rates, not part of the step."""
    import torch
    import torch.nn.functional as F
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(7)
    shapes = {"gate_up": (512, 16384, 3072), "down": (512, 3072, 8192),
              "qkv": (512, 5120, 3072), "wo": (512, 3072, 3072),
              # the 8B-shaped layer at 4096 tokens (QKV with biases: 6144 wide)
              "8b_gate_up": (4096, 28672, 4096), "8b_down": (4096, 4096, 14336),
              "8b_qkv": (4096, 6144, 4096), "8b_wo": (4096, 4096, 4096)}
    out = {}
    for name, (m, n, k) in shapes.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.float16, generator=g)
        row = {"m_n_k": [m, n, k]}
        for layout, shape, fn in (("w_kxn", (k, n), torch.matmul), ("w_nxk", (n, k), F.linear)):
            ws = [torch.randn(*shape, device="cuda", dtype=torch.float16, generator=g) for _ in range(4)]
            for w in ws:
                fn(a, w)
            torch.cuda.synchronize()
            reps = max(args.steps, 1) * (10 if m <= 512 else 2)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for i in range(reps):
                fn(a, ws[i % 4])
            end.record()
            torch.cuda.synchronize()
            us = start.elapsed_time(end) / reps * 1e3
            row[layout] = {"avg_us": round(us, 2), "tflops": round(2 * m * n * k / (us * 1e-6) / 1e12, 1)}
            del ws
        out[name] = row
        del a
    print(json.dumps({"library_gemms": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other prefill workloads (3B over a 1536-row prefix, 8B pp4096)")
    ap.add_argument("--secondary-only", choices=("prefix1536", "pp4096"),
                    help="time one secondary workload alone (profiling aid; no headline line)")
    ap.add_argument("--attn-form", choices=("auto", "one-head", "shared"), default="auto",
                    help="prefill attention kernel form (measurement aid; default: the automatic choice)")
    ap.add_argument("--breakdown", action="store_true",
                    help="also time every prefill kernel class per launch (HIP events)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="time the projection shapes of the 3B and 8B layers through torch's GEMMs and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this library runs on one GPU; the multi-GPU sharding "
                                   "is a design, not a launched path",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.secondary_only:
        secondary_only(args.secondary_only, args)
        return
    if args.library_gemms:
        library_gemms(args)
        return

    import torch
    import dense_decoder_layer_amd as ddl
    import synth
    from dense_decoder_layer_amd.workloads import DeviceStack

    cfg = synth.STACK_CONFIGS["llama3b_pp512"]
    torch.cuda.set_device(0)
    t0 = time.time()
    ctx = ddl.ddl_ctx_create(attn_form=ATTN_FORMS[args.attn_form])
    layers_iter = (synth.layer_weights(cfg, l) for l in range(cfg.n_layers))
    stack = DeviceStack(ctx, cfg, layers_iter)
    bufs = stack.buffers(cfg.batch, cfg.start_pos)
    hidden = torch.from_numpy(synth.hidden_rows(cfg)).cuda()
    torch.cuda.synchronize()
    log(f"packed {cfg.n_layers} layers in {time.time() - t0:.1f}s")

    for _ in range(args.warmup):
        assert stack.run(hidden, 0, None, None, bufs) == cfg.n_layers, ddl.ddl_last_error()
    ms, ms_med, ms_min = timed_steps(lambda: stack.run(hidden, 0, None, None, bufs), args.steps)
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (median {ms_med:.3f}, min {ms_min:.3f})")

    # second pass of the same steps: HIP events around every gate/up GEMM launch
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_GEMM_GATE_UP, args.steps * cfg.n_layers)
    for _ in range(args.steps):
        stack.run(hidden, 0, None, None, bufs)
    torch.cuda.synchronize()
    durs = ddl.ddl_probe_read(ctx, args.steps * cfg.n_layers)
    ddl.ddl_probe_enable(ctx, ddl.DDL_K_GEMM_GATE_UP, 0)
    gu_ms = sum(durs) / len(durs)

    breakdown = None
    if args.breakdown:
        kinds = {"rmsnorm": ddl.DDL_K_RMSNORM, "gemm_qkv": ddl.DDL_K_GEMM_QKV,
                 "qkv_post": ddl.DDL_K_QKV_POST, "attn_prefill": ddl.DDL_K_ATTN_PREFILL,
                 "gemm_wo": ddl.DDL_K_GEMM_WO, "gemm_gate_up": ddl.DDL_K_GEMM_GATE_UP,
                 "gemm_down": ddl.DDL_K_GEMM_DOWN}
        breakdown = {}
        for name, kind in kinds.items():
            cap = args.steps * cfg.n_layers * 2
            ddl.ddl_probe_enable(ctx, kind, cap)
            for _ in range(args.steps):
                stack.run(hidden, 0, None, None, bufs)
            torch.cuda.synchronize()
            d = ddl.ddl_probe_read(ctx, cap)
            ddl.ddl_probe_enable(ctx, kind, 0)
            breakdown[name] = {"avg_us": round(sum(d) / len(d) * 1e3, 2),
                               "per_step_us": round(sum(d) / args.steps * 1e3, 1)}
        log("per-kernel: " + json.dumps(breakdown))

    flops, gu_flops = algorithmic_flops(cfg)
    tok_s = cfg.batch / (ms / 1e3)
    achieved = gu_flops / (gu_ms / 1e3) / 1e12
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_median": round(ms_med, 4), "ms_min": round(ms_min, 4),
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
                     "traffic": gate_up_traffic()},
    }
    if breakdown:
        result["breakdown"] = breakdown
    if not args.no_secondary:
        result["secondary"] = secondary_bench(ddl, ctx, stack, hidden, args)
    del stack, bufs
    torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode layer at 32768 rows ...")
        result["decode"] = decode_bench(ddl, ctx)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg)
        # the same oracle beside the other workloads: the 3B stack over its
        # prefix (bounded like the headline's), the 8B stack on two layers
        # (extrapolated to 32), and one decode token
        for line, name, kw in zip(result.get("secondary", []),
                                  ("llama3b_prefix1536", "llama8b_pp4096_extras"),
                                  (dict(budget_s=8.0), dict(max_layers=2))):
            line["cpu_oracle"] = cpu_baseline(synth.STACK_CONFIGS[name], **kw)
        if "decode" in result:
            result["decode"]["cpu_oracle"] = cpu_baseline_decode()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

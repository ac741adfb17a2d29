"""GPU parity of ddl_prefill_dense_stack against the CPU oracle, on the same
seeded inputs, through the C ABI.  Tolerances (relative L2 over each array):
K/V rows of every layer <= 5e-3, final hidden <= 1e-2; run lengths, row
counts and declines exact."""
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

KV_TOL, HIDDEN_TOL = 5e-3, 1e-2


def rel(a, b) -> float:
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ddl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_decoder_layer_amd as m
    return m


def host_values(layers):
    for w in layers:
        yield {n: synth.values(a) for n, a in w.items()}


def gpu_run(ddl, cfg, inp, min_batch=1, hidden=None, attn_form=0):
    from dense_decoder_layer_amd.workloads import DeviceStack
    ctx = ddl.ddl_ctx_create(min_batch=min_batch, attn_form=attn_form)
    stack = DeviceStack(ctx, cfg, inp.layers)
    bufs = stack.buffers(cfg.batch, cfg.start_pos)
    h = torch.from_numpy(inp.hidden if hidden is None else hidden).cuda()
    pk = [torch.from_numpy(a).cuda() for a in inp.prefix_k] if cfg.start_pos else None
    pv = [torch.from_numpy(a).cuda() for a in inp.prefix_v] if cfg.start_pos else None
    run = stack.run(h, cfg.start_pos, pk, pv, bufs)
    torch.cuda.synchronize()
    out = bufs["hidden_out"].cpu().numpy()
    ks = [t.cpu().numpy() for t in bufs["k_rows"]]
    vs = [t.cpu().numpy() for t in bufs["v_rows"]]
    return run, out, ks, vs


def check_parity(name, cfg, inp, got, n_layers):
    run, out, ks, vs = got
    assert run == n_layers
    t0 = time.time()
    want, wk, wv = oracle.prefill_dense_stack(inp.hidden, host_values(inp.layers), cfg,
                                              cfg.start_pos, inp.prefix_k, inp.prefix_v)
    kv = [(rel(ks[l], wk[l]), rel(vs[l], wv[l])) for l in range(n_layers)]
    worst_kv = max(max(a, b) for a, b in kv)
    err_h = rel(out, want)
    row_err = np.linalg.norm(out - want, axis=1) / np.linalg.norm(want, axis=1)
    say(f"[{name}] oracle {time.time() - t0:.1f}s  K/V rel L2 max {worst_kv:.2e} "
        f"(layer0 {kv[0][0]:.2e}/{kv[0][1]:.2e}, last {kv[-1][0]:.2e}/{kv[-1][1]:.2e})  "
        f"hidden rel L2 {err_h:.2e}  worst token row {row_err.max():.2e}")
    assert ks[0].shape == (cfg.batch, cfg.kv_width)
    assert np.isfinite(out).all()
    assert worst_kv <= KV_TOL, kv
    assert err_h <= HIDDEN_TOL


def small(name, **kw):
    base = dict(name=name, n_layers=2, d_model=512, n_heads=8, n_kv_heads=2, head_dim=128,
                d_ff=1024, batch=150, start_pos=0, rope_theta=5e5, weight_dtype="bf16")
    base.update(kw)
    return synth.StackConfig(**base)


SMALL_CASES = {
    "tiny": synth.STACK_CONFIGS["tiny"],
    "tiny-b1": synth.STACK_CONFIGS["tiny"].replace(batch=1),
    "tiny-b3": synth.STACK_CONFIGS["tiny"].replace(batch=3),
    "tiny-b200-prefix37": synth.STACK_CONFIGS["tiny"].replace(batch=200, start_pos=37),
    "hd128-b150": small("hd128-b150"),
    "hd128-prefix100-b77": small("hd128-prefix100-b77", batch=77, start_pos=100),
    "hd128-extras": small("hd128-extras", batch=65, start_pos=37, qkv_bias=True, qk_norm=True,
                          softcap=30.0, gated=True, n_layers=3),
    "mha-hd64": small("mha-hd64", n_heads=4, n_kv_heads=4, head_dim=64, batch=130),
    "group4-hd128": small("group4-hd128", n_heads=16, n_kv_heads=4, d_model=1024, batch=129,
                          start_pos=200, d_ff=2816),
    "group3-fp32": small("group3-fp32", n_heads=6, n_kv_heads=2, d_model=768, batch=96,
                         weight_dtype="fp32", softcap=5.0),
    # eight query heads per KV head, softcap, a ragged batch over a prefix
    "group8-softcap-b333-prefix64": small("group8-softcap-b333-prefix64", n_heads=16,
                                          n_kv_heads=2, d_model=1024, batch=333, start_pos=64,
                                          softcap=50.0, d_ff=1536),
    # head_dim 64 with a prefix and the output gate
    "hd64-gated-prefix40": small("hd64-gated-prefix40", n_heads=8, n_kv_heads=4, head_dim=64,
                                 batch=45, start_pos=40, gated=True),
    # fewer new tokens than one 32-key tile, over a prefix that is not tile-aligned
    "b5-prefix70": small("b5-prefix70", batch=5, start_pos=70),
    # the 3B layer width and heads, a ragged batch over a ragged prefix
    "llama3b-2layers-b300-prefix777": synth.STACK_CONFIGS["llama3b_pp512"].replace(
        n_layers=2, batch=300, start_pos=777),
    # gated and soft-capped at the 3B width: the stacked q/k/v/gate projection
    # is split over K, so the gate columns get their partial sums added
    "llama3b-gated-softcap-2layers-b256": synth.STACK_CONFIGS["llama3b_pp512"].replace(
        n_layers=2, batch=256, gated=True, softcap=30.0),
    # RoPE variants: adjacent-pair layout; a partial Neox width; a partial
    # adjacent-pair width with per-pair frequency factors and an attention factor
    "rope-norm-prefix50": small("rope-norm-prefix50", rope_layout="norm", batch=90, start_pos=50),
    "rope-neox-rot64": small("rope-neox-rot64", rope_rot_dim=64, batch=70, start_pos=33),
    "rope-norm-rot96-freq-mscale": small(
        "rope-norm-rot96-freq-mscale", rope_layout="norm", rope_rot_dim=96, rope_mscale=0.75,
        rope_freq_factors=tuple(1.0 + 0.25 * i for i in range(48)), batch=64, start_pos=100),
    "rope-hd64-norm-freq": small("rope-hd64-norm-freq", n_heads=8, n_kv_heads=4, head_dim=64,
                                 rope_layout="norm", rope_freq_factors=tuple([2.0] * 32),
                                 batch=40),
    # the GELU-gated FFN (fp32 and bf16 weights)
    "geglu-b100": small("geglu-b100", ffn_act="geglu", batch=100, start_pos=20),
    "geglu-fp32-extras": small("geglu-fp32-extras", ffn_act="geglu", weight_dtype="fp32",
                               qkv_bias=True, qk_norm=True, batch=48),
    # sliding windows: shorter than one key tile, not tile-aligned over a
    # prefix, with softcap and gate, and longer than every key (no effect)
    "window7-b80": small("window7-b80", window=7, batch=80),
    "window100-prefix300-gated": small("window100-prefix300-gated", window=100, batch=150,
                                       start_pos=300, gated=True, softcap=20.0, n_layers=3),
    "window33-group8-b333": small("window33-group8-b333", n_heads=16, n_kv_heads=2,
                                  d_model=1024, d_ff=1536, window=33, batch=333, start_pos=64),
    "window-longer-than-keys": small("window-longer-than-keys", window=4096, batch=60,
                                     start_pos=10),
    # sandwich norms (post-attention and post-FFN): alone over a prefix, with
    # the GELU FFN, window, softcap and gate, and at the 3B width where the
    # wo/down projections split over K and the run's last down projection
    # is finished by the closing norm
    "post-norms-prefix40": small("post-norms-prefix40", post_norms=True, batch=72, start_pos=40),
    "post-norms-geglu-window-softcap": small("post-norms-geglu-window-softcap", post_norms=True,
                                             ffn_act="geglu", window=48, softcap=30.0, gated=True,
                                             batch=130, n_layers=3),
    "post-norms-llama3b-2layers-b256": synth.STACK_CONFIGS["llama3b_pp512"].replace(
        n_layers=2, batch=256, post_norms=True),
    # more than 2048 new tokens, a ragged count: the large-M GEMM form for
    # the GELU FFN, and at hidden 4096 for SwiGLU and the residual
    # projections (wo with K 4096, down with a K of no straight-line form)
    "geglu-b2100": small("geglu-b2100", ffn_act="geglu", batch=2100),
    "wide-b2100": small("wide-b2100", d_model=4096, n_heads=32, n_kv_heads=8, d_ff=2048,
                        batch=2100, n_layers=1),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_stacks_match_oracle(ddl, name):
    cfg = SMALL_CASES[name]
    say(f"case {name}: B={cfg.batch} S={cfg.start_pos} L={cfg.n_layers} d={cfg.d_model} "
        f"heads={cfg.n_heads}/{cfg.n_kv_heads}x{cfg.head_dim}")
    inp = synth.stack_inputs(cfg)
    check_parity(name, cfg, inp, gpu_run(ddl, cfg, inp), cfg.n_layers)


# the same cases through the attention form where the query heads of a KV
# head share each K/V tile (the automatic choice takes it only on large
# grids); cases with one query head per KV head have no such form
SHARED_CASES = [n for n, c in SMALL_CASES.items() if c.n_heads > c.n_kv_heads]


@pytest.mark.parametrize("name", SHARED_CASES)
def test_small_stacks_shared_kv_tiles_match_oracle(ddl, name):
    cfg = SMALL_CASES[name]
    say(f"case {name} (shared K/V tiles)")
    inp = synth.stack_inputs(cfg)
    check_parity(name, cfg, inp, gpu_run(ddl, cfg, inp, attn_form=ddl.DDL_ATTN_SHARED),
                 cfg.n_layers)


def test_deterministic_and_causal(ddl):
    cfg = small("causal", batch=140, start_pos=20, softcap=20.0, gated=True)
    inp = synth.stack_inputs(cfg)
    a = gpu_run(ddl, cfg, inp)
    b = gpu_run(ddl, cfg, inp)
    assert np.array_equal(a[1], b[1]) and all(np.array_equal(x, y) for x, y in zip(a[2], b[2]))
    cut = 70
    pert = inp.hidden.copy()
    pert[cut:] += np.float32(3.0)
    c = gpu_run(ddl, cfg, inp, hidden=pert)
    assert np.array_equal(a[1][:cut], c[1][:cut])
    for l in range(cfg.n_layers):
        assert np.array_equal(a[2][l][:cut], c[2][l][:cut])
        assert np.array_equal(a[3][l][:cut], c[3][l][:cut])
    assert not np.allclose(a[1][cut:], c[1][cut:])


def test_position_zero_k_rows_are_unrotated(ddl):
    # with no prefix, token 0 sits at position 0 where RoPE is the identity:
    # its K row equals the same layer run without RoPE
    cfg = small("pos0", batch=4)
    inp = synth.stack_inputs(cfg)
    rot = gpu_run(ddl, cfg, inp)
    flat = gpu_run(ddl, cfg.replace(rope_theta=None), inp)
    assert np.array_equal(rot[2][0][0], flat[2][0][0])
    assert not np.array_equal(rot[2][0][1], flat[2][0][1])


def _sentinel_bufs(stack, batch):
    bufs = stack.buffers(batch)
    bufs["hidden_out"].fill_(7.0)
    for t in bufs["k_rows"] + bufs["v_rows"]:
        t.fill_(7.0)
    return bufs


def test_declines_touch_nothing_and_runs_stop_at_ineligible_layer(ddl):
    from dense_decoder_layer_amd.workloads import DeviceStack
    cfg = synth.STACK_CONFIGS["tiny"].replace(n_layers=3)
    inp = synth.stack_inputs(cfg)
    ctx = ddl.ddl_ctx_create()                   # min_batch 4
    stack = DeviceStack(ctx, cfg, inp.layers)
    h = torch.from_numpy(inp.hidden).cuda()
    untouched = lambda bufs, n: (bool((bufs["hidden_out"] == 7.0).all()) and
                                 all(bool((t == 7.0).all()) for t in bufs["k_rows"][:n]))
    # batch below min_batch
    bufs = _sentinel_bufs(stack, 3)
    assert stack.run(h[:3], 0, None, None, bufs) == ddl.DDL_DECLINED
    torch.cuda.synchronize()
    assert untouched(bufs, 3) and "min_batch" in ddl.ddl_last_error()
    # layer 0's cache rows differ from start_pos
    bufs = _sentinel_bufs(stack, 8)
    assert stack.run(h, 0, None, None, bufs, prefix_rows=[5, 0, 0]) == ddl.DDL_DECLINED
    torch.cuda.synchronize()
    assert untouched(bufs, 3)
    # layer 2 ineligible: the run is layers 0..1, layer 2's rows untouched
    bufs = _sentinel_bufs(stack, 8)
    assert stack.run(h, 0, None, None, bufs, prefix_rows=[0, 0, 9]) == 2
    torch.cuda.synchronize()
    assert bool((bufs["k_rows"][2] == 7.0).all()) and not bool((bufs["k_rows"][1] == 7.0).all())
    want, wk, _ = oracle.prefill_dense_stack(inp.hidden, list(host_values(inp.layers))[:2], cfg, 0)
    assert rel(bufs["hidden_out"].cpu().numpy(), want) <= HIDDEN_TOL
    # an injected failure after admission: error, nothing written
    fctx = ddl.ddl_ctx_create(fault_after_admission=True)
    bufs = _sentinel_bufs(stack, 8)
    with pytest.raises(RuntimeError, match="-3"):
        ddl.ddl_prefill_dense_stack(fctx, h, stack.layers, 0, None, None, [0, 0, 0],
                                    bufs["hidden_out"], bufs["k_rows"], bufs["v_rows"],
                                    bufs["workspace"])
    torch.cuda.synchronize()
    assert untouched(bufs, 3)
    # workspace too small
    bufs = _sentinel_bufs(stack, 8)
    with pytest.raises(RuntimeError, match="-4"):
        ddl.ddl_prefill_dense_stack(ctx, h, stack.layers, 0, None, None, [0, 0, 0],
                                    bufs["hidden_out"], bufs["k_rows"], bufs["v_rows"],
                                    bufs["workspace"][:100])
    # a layer the kernels do not serve is declined at pack time
    assert ddl.ddl_layer_pack(ctx, ddl.layer_desc(256, 4, 2, 64, 704, has_sinks=1), {},
                              ddl.DDL_DTYPE_F32, bufs["workspace"]) is None


def _full_case(ddl, name, cfg, n_layers=None):
    t0 = time.time()
    n = cfg.n_layers if n_layers is None else n_layers
    say(f"[{name}] drawing inputs for {n} layers ...")
    inp = synth.stack_inputs(cfg, n)
    say(f"[{name}] inputs {time.time() - t0:.1f}s; packing and running on the GPU ...")
    got = gpu_run(ddl, cfg.replace(n_layers=n), inp)
    say(f"[{name}] GPU done {time.time() - t0:.1f}s; oracle ...")
    check_parity(name, cfg, inp, got, n)


@pytest.mark.timeout(900)
def test_llama3b_pp512_full_stack(ddl):
    _full_case(ddl, "llama3b_pp512", synth.STACK_CONFIGS["llama3b_pp512"])


@pytest.mark.timeout(900)
def test_llama3b_prefix1536_full_stack(ddl):
    _full_case(ddl, "llama3b_prefix1536", synth.STACK_CONFIGS["llama3b_prefix1536"])


@pytest.fixture(scope="module")
def llama8b_gpu(ddl):
    """The whole 32-layer 8B-shaped stack with biases and QK norms at pp4096,
    run once on the GPU; the weights are drawn and packed one layer at a time."""
    from dense_decoder_layer_amd.workloads import DeviceStack
    cfg = synth.STACK_CONFIGS["llama8b_pp4096_extras"]
    t0 = time.time()
    say(f"[llama8b_pp4096_extras] packing {cfg.n_layers} layers ...")
    ctx = ddl.ddl_ctx_create()
    stack = DeviceStack(ctx, cfg, (synth.layer_weights(cfg, l) for l in range(cfg.n_layers)))
    bufs = stack.buffers(cfg.batch, 0)
    hidden = synth.hidden_rows(cfg)
    run = stack.run(torch.from_numpy(hidden).cuda(), 0, None, None, bufs)
    torch.cuda.synchronize()
    out = bufs["hidden_out"].cpu().numpy()
    ks = [t.cpu().numpy() for t in bufs["k_rows"]]
    vs = [t.cpu().numpy() for t in bufs["v_rows"]]
    say(f"[llama8b_pp4096_extras] GPU stack done in {time.time() - t0:.1f}s, run_len {run}")
    del stack, bufs
    torch.cuda.empty_cache()
    # the oracle's hidden entering each layer, filled chunk by chunk
    return {"cfg": cfg, "run": run, "out": out, "ks": ks, "vs": vs, "x": {0: hidden}}


LLAMA8B_CHUNK = 8


@pytest.mark.timeout(900)
@pytest.mark.parametrize("chunk", range(4))
def test_llama8b_pp4096_extras_full_stack(llama8b_gpu, chunk):
    # all 32 layers against the oracle, eight at a time: every layer's K/V
    # rows, and the final hidden after the last chunk
    st = llama8b_gpu
    cfg = st["cfg"]
    assert st["run"] == cfg.n_layers
    lo = chunk * LLAMA8B_CHUNK
    start = max(l for l in st["x"] if l <= lo)        # resume where the oracle stopped
    x = st["x"][start]
    for l in range(start, lo + LLAMA8B_CHUNK):
        t0 = time.time()
        w = {n: synth.values(a) for n, a in synth.layer_weights(cfg, l).items()}
        x, wk, wv = oracle.dense_layer(x, w, cfg, 0)
        st["x"][l + 1] = x
        if l < lo:
            continue
        ek, ev = rel(st["ks"][l], wk), rel(st["vs"][l], wv)
        say(f"[llama8b_pp4096_extras] layer {l}: K {ek:.2e} V {ev:.2e} "
            f"(oracle {time.time() - t0:.1f}s)")
        assert ek <= KV_TOL and ev <= KV_TOL
    if lo + LLAMA8B_CHUNK == cfg.n_layers:
        err = rel(st["out"], x)
        say(f"[llama8b_pp4096_extras] hidden after {cfg.n_layers} layers: {err:.2e}")
        assert np.isfinite(st["out"]).all() and err <= HIDDEN_TOL


def test_run_of_layers_with_different_options(ddl):
    # one run whose layers differ in everything that is per layer: RoPE
    # (Neox theta 5e5 / Norm theta 1e4 over 64 channels with factors / none),
    # FFN activation, window, softcap, sandwich norms.  The position
    # table is rebuilt whenever the RoPE description changes.  A fourth layer
    # with another rms_eps ends the run.
    base = small("mixed", n_layers=1, batch=70, start_pos=0, d_model=512, n_heads=8, n_kv_heads=2,
                 head_dim=128, d_ff=1024)
    cfgs = [base,
            base.replace(rope_layout="norm", rope_theta=1e4, rope_rot_dim=64,
                         rope_freq_factors=tuple(1.0 + 0.1 * i for i in range(32)),
                         ffn_act="geglu", window=20, softcap=15.0, post_norms=True),
            base.replace(rope_theta=None, gated=False, window=0, qk_norm=False),
            base.replace(rms_eps=1e-6)]
    from dense_decoder_layer_amd.workloads import desc_for
    ctx = ddl.ddl_ctx_create(min_batch=1)
    layers, host = [], []
    for i, c in enumerate(cfgs):
        w = synth.layer_weights(c.replace(seed=i), 0)
        host.append(w)
        layers.append(ddl.pack_layer_from_host(ctx, desc_for(c), w))
    B, kvw = base.batch, base.kv_width
    x = synth.hidden_rows(base)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty(B, base.d_model, **f32)
    ks = [torch.full((B, kvw), 7.0, **f32) for _ in cfgs]
    vs = [torch.full((B, kvw), 7.0, **f32) for _ in cfgs]
    ws = torch.empty(ddl.ddl_workspace_bytes(layers, B, 0), dtype=torch.uint8, device="cuda")
    run = ddl.ddl_prefill_dense_stack(ctx, torch.from_numpy(x).cuda(), layers, 0, None, None,
                                      [0] * len(cfgs), out, ks, vs, ws)
    torch.cuda.synchronize()
    assert run == 3, ddl.ddl_last_error()
    assert bool((ks[3] == 7.0).all())                 # the fourth layer did not run
    want = np.asarray(x, np.float64)
    for l in range(3):
        w = {n: synth.values(a) for n, a in host[l].items()}
        want, wk, wv = oracle.dense_layer(want, w, cfgs[l], 0)
        ek, ev = rel(ks[l].cpu().numpy(), wk), rel(vs[l].cpu().numpy(), wv)
        say(f"[mixed] layer {l}: K {ek:.2e} V {ev:.2e}")
        assert ek <= KV_TOL and ev <= KV_TOL
    err = rel(out.cpu().numpy(), want)
    say(f"[mixed] hidden after 3 layers: {err:.2e}")
    assert err <= HIDDEN_TOL

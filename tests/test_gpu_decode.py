"""GPU parity of ddl_attn_layer and ddl_decode_layer (one token against the
device KV mirror) with the CPU oracle, and the mirror's staleness and
capacity rules, through the C ABI.

The single-token path computes in fp32 throughout; its weights are the
packed fp16 matrices, which hold bf16 weights exactly.  So the output hidden
must match the oracle within relative L2 1e-4 for bf16 weights, and 2e-3 for
fp32 weights (rounded to fp16's 11-bit significand when packed).  At the
decode shapes the output is mostly residual and FFN, so one case removes
both (residual 0, down projection 0: the output is wo . attention) and holds
the attention's own contribution to the same bound.  The appended mirror
row, seq_len and declines are exact."""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-4      # fp32 arithmetic, weights exact
TOL_FP32W = 2e-3     # fp32 weights rounded to fp16 when packed


def tol_for(cfg) -> float:
    return TOL_BF16 if cfg.weight_dtype == "bf16" else TOL_FP32W


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


class Decode:
    """A packed layer, a mirror sized by the capacity policy, and buffers."""

    def __init__(self, ddl, cfg, inputs, ctx=None, planned=0):
        from dense_decoder_layer_amd.workloads import desc_for
        self.ddl, self.cfg, self.inp = ddl, cfg, inputs
        self.ctx = ctx or ddl.ddl_ctx_create()
        self.layer = ddl.pack_layer_from_host(self.ctx, desc_for(cfg.stack_view()),
                                              inputs["weights"])
        self.cap = ddl.ddl_mirror_plan_capacity(cfg.rows, planned)
        self.buf = torch.empty(ddl.ddl_mirror_bytes(cfg.n_kv_heads, cfg.head_dim, self.cap),
                               dtype=torch.uint8, device="cuda")
        self.mirror = ddl.ddl_mirror_init(self.buf, cfg.n_kv_heads, cfg.head_dim, self.cap)
        self.ws = torch.empty(ddl.ddl_attn_workspace_bytes(self.layer, self.cap),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty(cfg.d_model, dtype=torch.float32, device="cuda")

    def upload(self, k, v, rows):
        return self.ddl.ddl_mirror_upload(self.mirror, torch.from_numpy(k).cuda(),
                                          torch.from_numpy(v).cuda(), rows)

    def step(self, rows, q, k, v, gate, residual, ctx=None):
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        rc = self.ddl.ddl_attn_layer(ctx or self.ctx, self.mirror, rows, t(q), t(k), t(v),
                                     t(gate), self.cfg.n_heads, self.cfg.softcap, self.layer,
                                     t(residual), self.out, self.ws)
        torch.cuda.synchronize()
        return rc

    def mirror_rows(self, rows):
        kvw = self.cfg.kv_width
        flat = self.buf.view(torch.float32)
        half = flat.numel() // 2
        return (flat[: rows * kvw].view(rows, kvw).cpu().numpy(),
                flat[half: half + rows * kvw].view(rows, kvw).cpu().numpy())


def weights_values(inp):
    return {n: synth.values(a) for n, a in inp["weights"].items()}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("rows", synth.DECODE_ROWS)
def test_attn_layer_dec_sweep(ddl, rows):
    # the decode workload: 32 q / 8 KV heads x 128, softcap 50, sigmoid gate,
    # hidden 4096, SwiGLU 14336, at every swept context length
    cfg = synth.DECODE_CONFIG.replace(rows=rows)
    say(f"[attn_layer dec sweep] rows={rows} hq={cfg.n_heads} hkv={cfg.n_kv_heads} "
        f"d={cfg.d_model} f={cfg.d_ff}")
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    assert dec.upload(inp["cache_k"], inp["cache_v"], rows) == 1
    assert ddl.ddl_mirror_seq_len(dec.mirror) == rows
    rc = dec.step(rows, inp["q"], inp["k"], inp["v"], inp["gate"], inp["residual"])
    assert rc == 1, ddl.ddl_last_error()
    assert ddl.ddl_mirror_seq_len(dec.mirror) == rows + 1
    mk, mv = dec.mirror_rows(rows + 1)
    assert np.array_equal(mk[rows], inp["k"]) and np.array_equal(mv[rows], inp["v"])
    assert np.array_equal(mk[:rows], inp["cache_k"]) and np.array_equal(mv[:rows], inp["cache_v"])
    t0 = time.time()
    want = oracle.attn_layer(inp["q"], inp["k"], inp["v"], inp["gate"], inp["cache_k"],
                             inp["cache_v"], rows, weights_values(inp), cfg, inp["residual"])
    err = rel(dec.out.cpu().numpy(), want)
    say(f"  oracle {time.time() - t0:.1f}s out rel L2 {err:.2e}")
    assert err <= TOL_BF16


@pytest.mark.timeout(300)
@pytest.mark.parametrize("rows", synth.DECODE_ROWS)
def test_attn_layer_dec_attention_only(ddl, rows):
    # residual 0 and down projection 0: out = wo . (sigmoid(gate) * attention),
    # so the check sees the attention itself, not the residual stream
    cfg = synth.DECODE_CONFIG.replace(rows=rows)
    say(f"[attn_layer attention-only] rows={rows}")
    inp = synth.decode_inputs(cfg)
    inp["weights"] = dict(inp["weights"])
    inp["weights"]["wd"] = np.zeros_like(inp["weights"]["wd"])
    zero = np.zeros(cfg.d_model, np.float32)
    dec = Decode(ddl, cfg, inp)
    assert dec.upload(inp["cache_k"], inp["cache_v"], rows) == 1
    assert dec.step(rows, inp["q"], inp["k"], inp["v"], inp["gate"], zero) == 1
    w = weights_values(inp)
    want = oracle.attn_layer(inp["q"], inp["k"], inp["v"], inp["gate"], inp["cache_k"],
                             inp["cache_v"], rows, w, cfg, zero)
    got = dec.out.cpu().numpy()
    err = rel(got, want)
    # every bit of this output comes from the attention: without it (o = 0)
    # the output would be exactly zero
    say(f"  out rel L2 {err:.2e}  |out| {np.linalg.norm(want):.3e}")
    assert np.linalg.norm(want) > 0 and err <= TOL_BF16


def small_cfg(**kw):
    base = dict(name="small-decode", d_model=512, n_heads=8, n_kv_heads=2, head_dim=128,
                d_ff=1024, rows=100, softcap=0.0, gated=False)
    base.update(kw)
    return synth.DecodeConfig(**base)


@pytest.mark.parametrize("kw", [dict(), dict(gated=True, softcap=2.0),
                                dict(n_heads=4, n_kv_heads=4, head_dim=64, rows=0),
                                dict(n_heads=6, n_kv_heads=2, rows=1000, weight_dtype="fp32"),
                                dict(n_heads=16, n_kv_heads=2, rows=17),
                                # KV row widths the row-per-wave kernel does not
                                # take (128 floats) and the widths it does at
                                # other group sizes
                                dict(n_heads=4, n_kv_heads=1, rows=700, softcap=10.0),
                                dict(n_heads=8, n_kv_heads=8, rows=333, gated=True),
                                dict(n_heads=16, n_kv_heads=16, head_dim=64, rows=65),
                                # the GELU-gated FFN in the decode tail
                                dict(ffn_act="geglu", rows=257, gated=True, softcap=30.0)])
def test_decode_shapes(ddl, kw):
    cfg = small_cfg(**kw)
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    dec.upload(inp["cache_k"], inp["cache_v"], cfg.rows)
    gate = inp["gate"] if cfg.gated else None
    assert dec.step(cfg.rows, inp["q"], inp["k"], inp["v"], gate, inp["residual"]) == 1
    want = oracle.attn_layer(inp["q"], inp["k"], inp["v"], gate, inp["cache_k"], inp["cache_v"],
                             cfg.rows, weights_values(inp), cfg, inp["residual"])
    err = rel(dec.out.cpu().numpy(), want)
    say(f"decode {kw}: out rel L2 {err:.2e}")
    assert err <= tol_for(cfg)


def test_decode_chain_and_mirror_rules(ddl):
    cfg = small_cfg(rows=40, gated=True, softcap=50.0)
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    w = weights_values(inp)
    host_k, host_v = inp["cache_k"].copy(), inp["cache_v"].copy()
    rng = np.random.default_rng(5)
    # stale mirror (never uploaded: seq_len 0 != 40) declines and touches nothing
    assert dec.step(40, inp["q"], inp["k"], inp["v"], inp["gate"], inp["residual"]) == 0
    assert ddl.ddl_mirror_seq_len(dec.mirror) == 0 and "stale" in ddl.ddl_last_error()
    dec.upload(host_k, host_v, 40)
    for step in range(4):
        rows = host_k.shape[0]
        q, k, v, gate, x = (rng.standard_normal(n).astype(np.float32) for n in
                            (cfg.q_width, cfg.kv_width, cfg.kv_width, cfg.q_width, cfg.d_model))
        assert dec.step(rows, q, k, v, gate, x) == 1, ddl.ddl_last_error()
        want = oracle.attn_layer(q, k, v, gate, host_k, host_v, rows, w, cfg, x)
        assert rel(dec.out.cpu().numpy(), want) <= TOL_BF16
        host_k, host_v = np.vstack([host_k, k]), np.vstack([host_v, v])   # the caller's push
        assert ddl.ddl_mirror_seq_len(dec.mirror) == host_k.shape[0]
    # the host cache moves backwards: the mirror is stale, declines, re-uploads
    host_k, host_v = host_k[:30], host_v[:30]
    assert dec.step(30, inp["q"], inp["k"], inp["v"], inp["gate"], inp["residual"]) == 0
    dec.upload(host_k, host_v, 30)
    assert dec.step(30, inp["q"], inp["k"], inp["v"], inp["gate"], inp["residual"]) == 1
    want = oracle.attn_layer(inp["q"], inp["k"], inp["v"], inp["gate"], host_k, host_v, 30, w,
                             cfg, inp["residual"])
    assert rel(dec.out.cpu().numpy(), want) <= TOL_BF16
    # an injected failure after admission marks the mirror stale
    fctx = ddl.ddl_ctx_create(fault_after_admission=True)
    with pytest.raises(RuntimeError, match="-3"):
        dec.step(31, inp["q"], inp["k"], inp["v"], inp["gate"], inp["residual"], ctx=fctx)
    assert ddl.ddl_mirror_seq_len(dec.mirror) == -1


def test_capacity_rule(ddl):
    cfg = small_cfg(rows=511)
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    assert dec.cap == 512
    dec.upload(inp["cache_k"], inp["cache_v"], 511)
    assert dec.step(511, inp["q"], inp["k"], inp["v"], None, inp["residual"]) == 1
    # 512 rows fill the mirror: the next token needs a bigger one
    assert dec.step(512, inp["q"], inp["k"], inp["v"], None, inp["residual"]) == 0
    assert "capacity" in ddl.ddl_last_error()
    assert ddl.ddl_mirror_plan_capacity(512) == 1024
    assert ddl.ddl_mirror_plan_capacity(512, 2048) == 2048


def test_windowed_layer_is_declined_untouched(ddl):
    # a sliding-window layer is not served by the single-token path: declined
    # before any device work, the mirror keeps its rows and seq_len
    from dense_decoder_layer_amd.workloads import desc_for
    cfg = small_cfg(rows=50)
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    dec.layer = ddl.pack_layer_from_host(dec.ctx, desc_for(cfg.stack_view().replace(window=16)),
                                         inp["weights"])
    assert dec.upload(inp["cache_k"], inp["cache_v"], cfg.rows) == 1
    dec.out.fill_(7.0)
    rc = dec.step(cfg.rows, inp["q"], inp["k"], inp["v"], None, inp["residual"])
    assert rc == 0 and "window" in ddl.ddl_last_error()
    assert ddl.ddl_mirror_seq_len(dec.mirror) == cfg.rows
    assert torch.all(dec.out == 7.0)
    k, _ = dec.mirror_rows(cfg.rows)
    np.testing.assert_array_equal(k, inp["cache_k"][: cfg.rows])


def test_sandwich_norm_layer_is_declined_untouched(ddl):
    from dense_decoder_layer_amd.workloads import desc_for
    cfg = small_cfg(rows=20)
    inp = synth.decode_inputs(cfg)
    dec = Decode(ddl, cfg, inp)
    w = dict(inp["weights"])
    w["g_post_attn"] = np.ones(cfg.d_model, np.float32)
    w["g_post_ffn"] = np.ones(cfg.d_model, np.float32)
    dec.layer = ddl.pack_layer_from_host(dec.ctx, desc_for(cfg.stack_view().replace(post_norms=True)),
                                         w)
    assert dec.upload(inp["cache_k"], inp["cache_v"], cfg.rows) == 1
    dec.out.fill_(7.0)
    assert dec.step(cfg.rows, inp["q"], inp["k"], inp["v"], None, inp["residual"]) == 0
    assert "post" in ddl.ddl_last_error()
    assert ddl.ddl_mirror_seq_len(dec.mirror) == cfg.rows and torch.all(dec.out == 7.0)


# ---------------------------------------------------------------------------
# ddl_decode_layer: the whole single-token layer (head on the device)

def dl_cfg(name, **kw):
    base = dict(name=name, n_layers=1, d_model=512, n_heads=8, n_kv_heads=2, head_dim=128,
                d_ff=1024, batch=1, start_pos=100, rope_theta=5e5, weight_dtype="bf16")
    base.update(kw)
    return synth.StackConfig(**base)


DECODE_LAYER_CASES = {
    "llama3b-rows1000-gated-softcap": synth.STACK_CONFIGS["llama3b_pp512"].replace(
        n_layers=1, batch=1, start_pos=1000, gated=True, softcap=50.0),
    "llama8b-extras-rows4096": synth.STACK_CONFIGS["llama8b_pp4096_extras"].replace(
        n_layers=1, batch=1, start_pos=4096),
    "all-options-rows77": dl_cfg("all-options-rows77", start_pos=77, qkv_bias=True, qk_norm=True,
                                 gated=True, softcap=20.0, rope_layout="norm", rope_rot_dim=96,
                                 rope_freq_factors=tuple(1.0 + 0.5 * i for i in range(48)),
                                 rope_mscale=0.9, ffn_act="geglu"),
    "mha-hd64-first-token": dl_cfg("mha-hd64-first-token", n_heads=4, n_kv_heads=4, head_dim=64,
                                   start_pos=0, weight_dtype="fp32"),
    "neox-rot64-rows300": dl_cfg("neox-rot64-rows300", rope_rot_dim=64, start_pos=300),
}


class DecodeLayer:
    def __init__(self, ddl, cfg, planned=0):
        from dense_decoder_layer_amd.workloads import desc_for
        self.ddl, self.cfg = ddl, cfg
        self.inp = synth.stack_inputs(cfg)
        self.ctx = ddl.ddl_ctx_create()
        self.layer = ddl.pack_layer_from_host(self.ctx, desc_for(cfg), self.inp.layers[0])
        rows = cfg.start_pos
        self.cap = ddl.ddl_mirror_plan_capacity(rows, planned)
        self.buf = torch.empty(ddl.ddl_mirror_bytes(cfg.n_kv_heads, cfg.head_dim, self.cap),
                               dtype=torch.uint8, device="cuda")
        self.mirror = ddl.ddl_mirror_init(self.buf, cfg.n_kv_heads, cfg.head_dim, self.cap)
        if rows:
            assert ddl.ddl_mirror_upload(self.mirror, torch.from_numpy(self.inp.prefix_k[0]).cuda(),
                                         torch.from_numpy(self.inp.prefix_v[0]).cuda(), rows) == 1
        self.ws = torch.empty(ddl.ddl_attn_workspace_bytes(self.layer, self.cap),
                              dtype=torch.uint8, device="cuda")
        f32 = dict(dtype=torch.float32, device="cuda")
        self.out = torch.empty(cfg.d_model, **f32)
        self.k_row = torch.empty(cfg.kv_width, **f32)
        self.v_row = torch.empty(cfg.kv_width, **f32)

    def step(self, rows, x):
        rc = self.ddl.ddl_decode_layer(self.ctx, self.mirror, rows,
                                       torch.from_numpy(np.ascontiguousarray(x)).cuda(),
                                       self.layer, self.out, self.k_row, self.v_row, self.ws)
        torch.cuda.synchronize()
        return rc

    def mirror_row(self, r):
        kvw = self.cfg.kv_width
        flat = self.buf.view(torch.float32)
        half = flat.numel() // 2
        return (flat[r * kvw:(r + 1) * kvw].cpu().numpy(),
                flat[half + r * kvw: half + (r + 1) * kvw].cpu().numpy())


@pytest.mark.parametrize("name", list(DECODE_LAYER_CASES))
def test_decode_layer_matches_oracle(ddl, name):
    cfg = DECODE_LAYER_CASES[name]
    say(f"[decode_layer {name}] rows={cfg.start_pos}")
    dl = DecodeLayer(ddl, cfg)
    rows, x = cfg.start_pos, dl.inp.hidden[0]
    assert dl.step(rows, x) == 1
    assert ddl.ddl_mirror_seq_len(dl.mirror) == rows + 1
    w = {n: synth.values(a) for n, a in dl.inp.layers[0].items()}
    ck = dl.inp.prefix_k[0] if rows else np.zeros((0, cfg.kv_width), np.float32)
    cv = dl.inp.prefix_v[0] if rows else np.zeros((0, cfg.kv_width), np.float32)
    want, wk, wv = oracle.decode_layer(x, w, cfg, ck, cv, rows)
    got_k, got_v = dl.k_row.cpu().numpy(), dl.v_row.cpu().numpy()
    err, ek, ev = rel(dl.out.cpu().numpy(), want), rel(got_k, wk), rel(got_v, wv)
    say(f"  out rel L2 {err:.2e}  k_row {ek:.2e}  v_row {ev:.2e}")
    assert err <= tol_for(cfg) and ek <= tol_for(cfg) and ev <= tol_for(cfg)
    mk, mv = dl.mirror_row(rows)            # the appended row is the returned row, bit for bit
    np.testing.assert_array_equal(mk, got_k)
    np.testing.assert_array_equal(mv, got_v)


def test_decode_layer_chain_and_declines(ddl):
    # two consecutive tokens: the second attends over the first one's row;
    # a stale row count is declined with nothing touched
    cfg = dl_cfg("chain", start_pos=40, gated=True, softcap=30.0, qk_norm=True)
    dl = DecodeLayer(ddl, cfg)
    w = {n: synth.values(a) for n, a in dl.inp.layers[0].items()}
    ck, cv = dl.inp.prefix_k[0], dl.inp.prefix_v[0]
    x0 = dl.inp.hidden[0]
    x1 = np.random.default_rng(5).standard_normal(cfg.d_model).astype(np.float32)
    assert dl.step(40, x0) == 1
    k0, v0 = dl.k_row.cpu().numpy(), dl.v_row.cpu().numpy()
    ck, cv = np.concatenate([ck, k0[None]]), np.concatenate([cv, v0[None]])
    dl.out.fill_(7.0)
    assert dl.step(40, x1) == 0 and "stale" in ddl.ddl_last_error()   # rows must be 41 now
    assert torch.all(dl.out == 7.0) and ddl.ddl_mirror_seq_len(dl.mirror) == 41
    assert dl.step(41, x1) == 1
    want, wk, _ = oracle.decode_layer(x1, w, cfg, ck, cv, 41)
    assert rel(dl.out.cpu().numpy(), want) <= TOL_BF16
    assert rel(dl.k_row.cpu().numpy(), wk) <= TOL_BF16
    assert ddl.ddl_mirror_seq_len(dl.mirror) == 42


# ---------------------------------------------------------------------------
# the decode step captured once as a HIP graph and replayed per token

def test_decode_graph_replays_match_eager_steps_and_oracle(ddl):
    cfg = dl_cfg("graph-chain", start_pos=40, gated=True, softcap=30.0, qk_norm=True,
                 qkv_bias=True)
    say("[decode graph] capture, 4 replays, an eager step, a rewind")
    g_side = DecodeLayer(ddl, cfg)           # the graph's mirror
    e_side = DecodeLayer(ddl, cfg)           # eager ddl_decode_layer on a second mirror
    w = {n: synth.values(a) for n, a in g_side.inp.layers[0].items()}
    f32 = dict(dtype=torch.float32, device="cuda")
    hidden = torch.empty(cfg.d_model, **f32)
    out, k_row, v_row = (torch.empty(n, **f32) for n in (cfg.d_model, cfg.kv_width, cfg.kv_width))
    ws = torch.empty_like(g_side.ws)
    graph = ddl.ddl_decode_graph_create(g_side.ctx, g_side.mirror, g_side.layer, hidden, out,
                                        k_row, v_row, ws)
    assert graph is not None, ddl.ddl_last_error()
    host_k, host_v = g_side.inp.prefix_k[0].copy(), g_side.inp.prefix_v[0].copy()
    rng = np.random.default_rng(11)

    def replay_and_check(rows, x, tag):
        hidden.copy_(torch.from_numpy(x))
        out.fill_(7.0)
        assert ddl.ddl_decode_graph_launch(g_side.ctx, graph, rows) == 1, ddl.ddl_last_error()
        torch.cuda.synchronize()
        want, wk, wv = oracle.decode_layer(x, w, cfg, host_k, host_v, rows)
        got = out.cpu().numpy()
        err, ek = rel(got, want), rel(k_row.cpu().numpy(), wk)
        say(f"  {tag} rows={rows}: out rel L2 {err:.2e}  k_row {ek:.2e}")
        assert err <= TOL_BF16 and ek <= TOL_BF16 and rel(v_row.cpu().numpy(), wv) <= TOL_BF16
        assert ddl.ddl_mirror_seq_len(g_side.mirror) == rows + 1
        mk, mv = g_side.mirror_row(rows)      # the appended row is the returned row
        np.testing.assert_array_equal(mk, k_row.cpu().numpy())
        np.testing.assert_array_equal(mv, v_row.cpu().numpy())
        return got

    for step in range(4):
        rows = host_k.shape[0]
        x = rng.standard_normal(cfg.d_model).astype(np.float32)
        got = replay_and_check(rows, x, f"replay {step}")
        # eager work between replays: the same token through ddl_decode_layer
        assert e_side.step(rows, x) == 1
        np.testing.assert_array_equal(e_side.k_row.cpu().numpy(), k_row.cpu().numpy())
        assert rel(got, e_side.out.cpu().numpy()) <= TOL_BF16
        host_k = np.vstack([host_k, k_row.cpu().numpy()])
        host_v = np.vstack([host_v, v_row.cpu().numpy()])
    # an eager step on the graph's own mirror, then a replay: the device row
    # count catches up
    rows = host_k.shape[0]
    x = rng.standard_normal(cfg.d_model).astype(np.float32)
    assert g_side.step(rows, x) == 1
    host_k = np.vstack([host_k, g_side.k_row.cpu().numpy()])
    host_v = np.vstack([host_v, g_side.v_row.cpu().numpy()])
    replay_and_check(host_k.shape[0], rng.standard_normal(cfg.d_model).astype(np.float32),
                     "after an eager step")
    host_k = np.vstack([host_k, k_row.cpu().numpy()])
    host_v = np.vstack([host_v, v_row.cpu().numpy()])
    # a stale row count is declined with nothing touched
    out.fill_(7.0)
    assert ddl.ddl_decode_graph_launch(g_side.ctx, graph, 3) == 0
    torch.cuda.synchronize()
    assert "stale" in ddl.ddl_last_error() and bool((out == 7.0).all())
    # the host cache rewinds to 30 rows: re-upload, replay at 30
    host_k, host_v = host_k[:30].copy(), host_v[:30].copy()
    assert ddl.ddl_mirror_upload(g_side.mirror, torch.from_numpy(host_k).cuda(),
                                 torch.from_numpy(host_v).cuda(), 30) == 1
    replay_and_check(30, rng.standard_normal(cfg.d_model).astype(np.float32), "after a rewind")
    ddl.ddl_decode_graph_destroy(graph)


def test_decode_graph_at_the_decode_workload(ddl):
    # the decode workload's layer shape (32/8 heads x 128, hidden 4096, FFN
    # 14336, gated, softcap 50) over 4096 cached rows, three replays
    base = synth.DECODE_CONFIG
    cfg = synth.StackConfig("dec-graph", 1, base.d_model, base.n_heads, base.n_kv_heads,
                            base.head_dim, base.d_ff, batch=1, start_pos=4096, rope_theta=5e5,
                            gated=True, softcap=base.softcap)
    dl = DecodeLayer(ddl, cfg)
    w = {n: synth.values(a) for n, a in dl.inp.layers[0].items()}
    f32 = dict(dtype=torch.float32, device="cuda")
    hidden = torch.empty(cfg.d_model, **f32)
    out, k_row, v_row = (torch.empty(n, **f32) for n in (cfg.d_model, cfg.kv_width, cfg.kv_width))
    graph = ddl.ddl_decode_graph_create(dl.ctx, dl.mirror, dl.layer, hidden, out, k_row, v_row,
                                        dl.ws)
    host_k, host_v = dl.inp.prefix_k[0].copy(), dl.inp.prefix_v[0].copy()
    rng = np.random.default_rng(12)
    for step in range(3):
        rows = host_k.shape[0]
        x = rng.standard_normal(cfg.d_model).astype(np.float32)
        hidden.copy_(torch.from_numpy(x))
        assert ddl.ddl_decode_graph_launch(dl.ctx, graph, rows) == 1, ddl.ddl_last_error()
        torch.cuda.synchronize()
        want, wk, _ = oracle.decode_layer(x, w, cfg, host_k, host_v, rows)
        err = rel(out.cpu().numpy(), want)
        say(f"[decode graph 32/8x128] rows={rows}: out rel L2 {err:.2e}")
        assert err <= TOL_BF16 and rel(k_row.cpu().numpy(), wk) <= TOL_BF16
        host_k = np.vstack([host_k, k_row.cpu().numpy()])
        host_v = np.vstack([host_v, v_row.cpu().numpy()])

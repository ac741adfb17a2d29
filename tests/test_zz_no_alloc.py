"""ddl_attn_layer_noalloc (the decode attention layer with the library's
fixed device scratch instead of a caller workspace) against ddl_attn_layer
through the C ABI: two calls in a row, the second on a smaller layer and
fewer rows, each matching the workspace entry point's output and mirror
bookkeeping exactly; a layer whose scratch exceeds the fixed size is
refused before any device work."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_decoder_layer_amd as m
    return m


def _setup(ddl, cfg):
    from dense_decoder_layer_amd.workloads import desc_for
    inp = synth.decode_inputs(cfg)
    ctx = ddl.ddl_ctx_create()
    layer = ddl.pack_layer_from_host(ctx, desc_for(cfg.stack_view()), inp["weights"])
    cap = ddl.ddl_mirror_plan_capacity(cfg.rows)
    mirrors = []
    for _ in range(2):
        buf = torch.empty(ddl.ddl_mirror_bytes(cfg.n_kv_heads, cfg.head_dim, cap),
                          dtype=torch.uint8, device="cuda")
        m = ddl.ddl_mirror_init(buf, cfg.n_kv_heads, cfg.head_dim, cap)
        assert ddl.ddl_mirror_upload(m, torch.from_numpy(inp["cache_k"]).cuda(),
                                     torch.from_numpy(inp["cache_v"]).cuda(), cfg.rows) == 1
        mirrors.append((m, buf))
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = {n: t(inp[n]) for n in ("q", "k", "v", "residual")}
    args["gate"] = t(inp["gate"]) if cfg.gated else None
    return ctx, layer, mirrors, args, cap


def _compare(ddl, cfg):
    ctx, layer, mirrors, a, cap = _setup(ddl, cfg)
    (m_ws, buf_ws), (m_na, buf_na) = mirrors
    ws = torch.empty(ddl.ddl_attn_workspace_bytes(layer, cap), dtype=torch.uint8, device="cuda")
    out_ws = torch.full((cfg.d_model,), 7.0, device="cuda")
    out_na = torch.full((cfg.d_model,), 7.0, device="cuda")
    assert ddl.ddl_attn_layer(ctx, m_ws, cfg.rows, a["q"], a["k"], a["v"], a["gate"], cfg.n_heads,
                              cfg.softcap, layer, a["residual"], out_ws, ws) == 1
    assert ddl.ddl_attn_layer_noalloc(ctx, m_na, cfg.rows, a["q"], a["k"], a["v"], a["gate"],
                                      cfg.n_heads, cfg.softcap, layer, a["residual"], out_na) == 1
    torch.cuda.synchronize()
    got, want = out_na.cpu().numpy(), out_ws.cpu().numpy()
    err = float(np.linalg.norm(got.astype(np.float64) - want) / np.linalg.norm(want))
    print(f"[no-alloc {cfg.name} rows={cfg.rows}] rel L2 vs workspace entry point {err:.2e}, "
          f"bit-identical {np.array_equal(got, want)}", flush=True)
    assert err <= 1e-4
    assert ddl.ddl_mirror_seq_len(m_na) == ddl.ddl_mirror_seq_len(m_ws) == cfg.rows + 1
    kvw = cfg.kv_width * (cfg.rows + 1)
    half = buf_na.numel() // 8          # floats per K half of the mirror
    np.testing.assert_array_equal(buf_na.view(torch.float32)[:kvw].cpu().numpy(),
                                  buf_ws.view(torch.float32)[:kvw].cpu().numpy())
    np.testing.assert_array_equal(buf_na.view(torch.float32)[half:half + kvw].cpu().numpy(),
                                  buf_ws.view(torch.float32)[half:half + kvw].cpu().numpy())


def test_no_alloc_matches_workspace_entry_point_twice(ddl):
    # first the decode workload at 4096 rows, then a smaller layer over fewer
    # rows: the second call must not see the first call's scratch contents
    _compare(ddl, synth.DECODE_CONFIG.replace(rows=4096))
    _compare(ddl, synth.DecodeConfig("small-decode", d_model=512, n_heads=8, n_kv_heads=2,
                                     head_dim=128, d_ff=1024, rows=100, softcap=0.0,
                                     gated=False))


def test_no_alloc_refuses_a_layer_above_its_scratch(ddl):
    # 64 query heads of 128: the split partials alone take 8 MiB, above the
    # fixed scratch; refused with nothing enqueued, the mirror untouched
    cfg = synth.DecodeConfig("wide-decode", d_model=1024, n_heads=64, n_kv_heads=8,
                             head_dim=128, d_ff=1024, rows=10, softcap=0.0, gated=False)
    ctx, layer, mirrors, a, cap = _setup(ddl, cfg)
    assert ddl.ddl_attn_workspace_bytes(layer, cap) > ddl.DDL_NOALLOC_SCRATCH_BYTES
    m, _ = mirrors[0]
    out = torch.full((cfg.d_model,), 7.0, device="cuda")
    with pytest.raises(RuntimeError, match="-4"):
        ddl.ddl_attn_layer_noalloc(ctx, m, cfg.rows, a["q"], a["k"], a["v"], None, cfg.n_heads,
                                   cfg.softcap, layer, a["residual"], out)
    torch.cuda.synchronize()
    assert ddl.ddl_mirror_seq_len(m) == cfg.rows and bool((out == 7.0).all())

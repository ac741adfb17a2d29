"""CPU pin of the range the kernels assume for the activations they store as
fp16 (the MFMA operands): the normed rows h and h2, the rotated q and k, v,
the gated attention output o and the SwiGLU activations a.  fp16 overflows
above 65504; on the synthetic workloads (every layer of the Llama-3.2-3B-
shaped stack, the 8B-shaped layer with biases and QK norms)
each stays below 1/64 of that, so the fp16 stores neither overflow nor
saturate.  Inputs far outside these distributions (activations of order
1e3 and more in the projections' outputs) are outside what the build
assumes."""
import numpy as np
import pytest

import oracle
import synth

FP16_MAX = 65504.0


def stored_fp16_maxima(x, w, cfg, start_pos=0):
    """Largest |value| of each fp16-stored activation of one layer, from the
    oracle's own steps, and the layer output."""
    B = x.shape[0]
    pos = start_pos + np.arange(B)
    h = oracle.rms_norm(x, w["g_attn"], cfg.rms_eps)
    q, gate, k, v = oracle.project_qkv(h, w, cfg, pos)
    o = oracle.causal_gqa_attention(q, k, v, start_pos, cfg.softcap, gate)
    x1 = x + o.reshape(B, -1) @ np.asarray(w["wo"], np.float64).T
    h2 = oracle.rms_norm(x1, w["g_ffn"], cfg.rms_eps)
    g = h2 @ np.asarray(w["wg"], np.float64).T
    a = oracle.silu(g) * (h2 @ np.asarray(w["wu"], np.float64).T)
    out = x1 + a @ np.asarray(w["wd"], np.float64).T
    m = {n: float(np.abs(t).max()) for n, t in
         dict(h=h, q=q, k=k, v=v, o=o, h2=h2, a=a).items()}
    return m, out


def test_llama3b_stack_activations_fit_fp16():
    # every layer of the stack, on the first 128 of the 512 tokens' rows
    cfg = synth.STACK_CONFIGS["llama3b_pp512"].replace(batch=128)
    x = synth.hidden_rows(cfg).astype(np.float64)
    worst = {}
    for l in range(cfg.n_layers):
        w = {n: synth.values(a) for n, a in synth.layer_weights(cfg, l).items()}
        m, x = stored_fp16_maxima(x, w, cfg)
        for n, v in m.items():
            worst[n] = max(worst.get(n, 0.0), v)
    assert max(worst.values()) < FP16_MAX / 64, worst


def test_llama8b_extras_layer_activations_fit_fp16():
    cfg = synth.STACK_CONFIGS["llama8b_pp4096_extras"].replace(batch=256)
    x = synth.hidden_rows(cfg).astype(np.float64)
    w = {n: synth.values(a) for n, a in synth.layer_weights(cfg, 0).items()}
    m, _ = stored_fp16_maxima(x, w, cfg)
    assert max(m.values()) < FP16_MAX / 64, m

"""CPU check that the decode parity tolerance can see the attention, at the
decode workload (32 q / 8 KV heads x 128, softcap 50, sigmoid gate, hidden
4096, SwiGLU 14336) and every swept row count:
* on the whole layer's output, dropping the attention moves it by far more
  than the bound the GPU tests hold the library to;
* on the attention-only output (residual 0, down projection 0: out =
  wo . attention), so does leaving out the new row or one cached row."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_decode import TOL_BF16


def rel(a, b) -> float:
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b))


@pytest.fixture(scope="module")
def dec_inputs():
    cfg = synth.DECODE_CONFIG
    inp = synth.decode_inputs(cfg)
    return cfg, inp, {n: synth.values(a) for n, a in inp["weights"].items()}


@pytest.mark.parametrize("rows", synth.DECODE_ROWS)
def test_dropping_the_attention_fails_the_decode_tolerance(dec_inputs, rows):
    cfg, inp, w = dec_inputs
    cfg = cfg.replace(rows=rows)
    ck, cv, q, k, v, gate = (inp[n] for n in ("cache_k", "cache_v", "q", "k", "v", "gate"))
    want = oracle.attn_layer(q, k, v, gate, ck, cv, rows, w, cfg, inp["residual"])
    closed = np.full_like(gate, -np.inf)          # sigmoid(-inf) = 0: no attention output
    no_attn = oracle.attn_layer(q, k, v, closed, ck, cv, rows, w, cfg, inp["residual"])
    assert rel(no_attn, want) > 10 * TOL_BF16

    w0 = dict(w, wd=np.zeros_like(w["wd"]))
    zero = np.zeros(cfg.d_model)
    want = oracle.attn_layer(q, k, v, gate, ck, cv, rows, w0, cfg, zero)
    # the new row left out (the last cached row counted twice instead)
    stale = oracle.attn_layer(q, ck[rows - 1], cv[rows - 1], gate, ck, cv, rows, w0, cfg, zero)
    # the first cached row left out
    short = oracle.attn_layer(q, k, v, gate, ck[1:], cv[1:], rows - 1, w0, cfg, zero)
    assert rel(stale, want) > 10 * TOL_BF16
    assert rel(short, want) > 10 * TOL_BF16

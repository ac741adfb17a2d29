"""The bench's algorithmic work per step, against the figures the workload
definitions fix: GEMM flops 2*B*params*L plus the unmasked causal triangle
4*hd*Hq*sum_b(S+b+1)*L (masked halves of diagonal tiles not counted)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def brute_flops(cfg):
    d, f, hd = cfg.d_model, cfg.d_ff, cfg.head_dim
    q, kv = cfg.n_heads * hd, cfg.n_kv_heads * hd
    per_token = 0
    # every projection as an explicit matrix: q, k, v (and gate), o, gate, up, down
    mats = [(q, d), (kv, d), (kv, d), (d, q), (f, d), (f, d), (d, f)]
    if cfg.gated:
        mats.append((q, d))
    for n_out, n_in in mats:
        per_token += 2 * n_out * n_in
    attn = 0
    for b in range(cfg.batch):
        keys = cfg.start_pos + b + 1          # causal: this token's prefix and itself
        attn += cfg.n_heads * keys * hd * 2 * 2   # q.k and p.v, a multiply and an add each
    return (per_token * cfg.batch + attn) * cfg.n_layers


@pytest.mark.parametrize("name,tflop", [("llama3b_pp512", 2.9314), ("llama3b_prefix1536", 3.2020),
                                        ("llama8b_pp4096_extras", 61.5737)])
def test_algorithmic_flops_per_step(name, tflop):
    cfg = synth.STACK_CONFIGS[name]
    flops, gate_up = bench.algorithmic_flops(cfg)
    assert flops == brute_flops(cfg)
    assert abs(flops / 1e12 - tflop) < 5e-5
    # the roofline kernel: one gate/up launch, 2 * B * (2F) * d
    assert gate_up == 2 * cfg.batch * 2 * cfg.d_ff * cfg.d_model


def test_gate_up_traffic_reads_the_committed_summary():
    # the committed counter summary carries the GEMM source's digest; the
    # bench reports its bytes only while they match
    t = bench.gate_up_traffic()
    assert t is None or 100e6 < t < 200e6

"""Writes tiny_stack_sample.json: sampled oracle outputs of the tiny stack
(2 layers, hidden 256, 4/2 heads of 64, FFN 704, 8 tokens, seed 0).

The pages print no worked example, so this fixture is a regression pin of the
oracle against its own committed past (it catches accidental edits), not a
correctness pin; the correctness pins are in test_oracle_pins.py.  It calls
only oracle/ and synth/.  Run from the repository root:
    python tests/golden/make_tiny_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ROWS = (0, 3, 7)
COLS = (0, 1, 100, 127)


def sample():
    cfg = synth.STACK_CONFIGS["tiny"]
    inp = synth.stack_inputs(cfg)
    layers = [{n: synth.values(a) for n, a in w.items()} for w in inp.layers]
    out, ks, vs = oracle.prefill_dense_stack(inp.hidden, layers, cfg, 0)
    return {
        "config": "tiny (seed 0)",
        "hidden_out": [[float(out[r, c]) for c in COLS] for r in ROWS],
        "k_rows_layer1": [[float(ks[1][r, c]) for c in COLS] for r in ROWS],
        "v_rows_layer0": [[float(vs[0][r, c]) for c in COLS] for r in ROWS],
        "rows": ROWS, "cols": COLS,
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_stack_sample.json")
    with open(path, "w") as f:
        json.dump(sample(), f, indent=1)
    print("wrote", path)

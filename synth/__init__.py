"""Seeded synthetic inputs for the dense decoder-layer stack.

This module is shared by the tests, the benchmark and the oracle's
callers.  It holds shapes, seeds and random draws only: none of the
layer's arithmetic lives here.  Every tensor is drawn from its own
counter-based stream (numpy's Philox4x64-10 bit generator keyed by
``(seed, stream_id)``, normals through ``Generator.standard_normal``), so a
tensor can be drawn on its own, in any order, on any thread, and always
comes out the same.

Distributions (a stated reading: the pages fix none):
  * projection matrices and biases  ~ N(0, 0.02)
  * RMSNorm / QK-norm / post-norm gains ~ 1 + N(0, 0.02)
  * hidden rows and prefix K/V rows ~ N(0, 1), fp32
  * decode-step q, k, v and gate    ~ N(0, 1), fp32
  * in a bf16 configuration the matrices are rounded to bf16 with
    round-to-nearest-even and kept as their 16-bit patterns; vectors stay
    fp32.

Matrices are row-major ``[out, in]``; activations are token-major.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "StackConfig", "DecodeConfig", "STACK_CONFIGS", "DECODE_CONFIG",
    "stack_inputs", "layer_weights", "hidden_rows", "prefix_rows",
    "decode_inputs", "to_bf16_bits", "bf16_bits_to_f32", "values",
    "MATRICES", "VECTORS",
]

# Stream ids of the per-layer tensors; the listing order is the draw order.
_SLOTS = {
    "g_attn": 0, "wq": 1, "wk": 2, "wv": 3, "bq": 4, "bk": 5, "bv": 6,
    "q_norm": 7, "k_norm": 8, "wo": 9, "g_ffn": 10, "wg": 11, "wu": 12,
    "wd": 13, "g_post_attn": 14, "g_post_ffn": 15, "prefix_k": 20, "prefix_v": 21,
}
MATRICES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
VECTORS = ("g_attn", "bq", "bk", "bv", "q_norm", "k_norm", "g_ffn", "g_post_attn", "g_post_ffn")
_HIDDEN_STREAM = 1
_DECODE_STREAM_BASE = 1 << 20


@dataclasses.dataclass(frozen=True)
class StackConfig:
    """Shape and options of one prefill workload (a run of dense layers)."""
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    batch: int
    start_pos: int
    rope_theta: float
    weight_dtype: str = "bf16"          # "bf16" or "fp32"
    rms_eps: float = 1e-5
    qkv_bias: bool = False
    qk_norm: bool = False
    softcap: float = 0.0                # 0 = no logit softcap
    gated: bool = False                 # double-width wq: [q ; gate]
    rope_layout: str = "neox"           # "neox" (half split) or "norm" (adjacent pairs)
    rope_rot_dim: int = 0               # rotated channels per head; 0 = head_dim
    rope_mscale: float = 1.0            # attention factor on the rotated channels
    rope_freq_factors: Optional[tuple] = None   # per-pair divisors of the frequency
    ffn_act: str = "swiglu"             # "swiglu" or "geglu" (gated GELU)
    window: int = 0                     # sliding window in keys; 0 = none
    post_norms: bool = False            # sandwich norms: post-attention and post-FFN gains
    seed: int = 0

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def shapes(self) -> Dict[str, tuple]:
        d, qw, kw, f = self.d_model, self.q_width, self.kv_width, self.d_ff
        s = {
            "g_attn": (d,),
            "wq": ((2 if self.gated else 1) * qw, d),
            "wk": (kw, d), "wv": (kw, d),
            "wo": (d, qw),
            "g_ffn": (d,),
            "wg": (f, d), "wu": (f, d), "wd": (d, f),
        }
        if self.qkv_bias:
            s.update(bq=(qw,), bk=(kw,), bv=(kw,))
        if self.qk_norm:
            s.update(q_norm=(self.head_dim,), k_norm=(self.head_dim,))
        if self.post_norms:
            s.update(g_post_attn=(d,), g_post_ffn=(d,))
        return s

    def replace(self, **kw) -> "StackConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One single-token attention layer against a device KV mirror."""
    name: str
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    rows: int                            # rows already in the cache/mirror
    softcap: float
    gated: bool
    weight_dtype: str = "bf16"
    rms_eps: float = 1e-5
    ffn_act: str = "swiglu"             # "swiglu" or "geglu" (gated GELU)
    seed: int = 0

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def stack_view(self) -> StackConfig:
        """The layer's weights drawn as a one-layer stack (so the packed
        layer format is shared with prefill)."""
        return StackConfig(
            name=self.name + "-layer", n_layers=1, d_model=self.d_model,
            n_heads=self.n_heads, n_kv_heads=self.n_kv_heads,
            head_dim=self.head_dim, d_ff=self.d_ff, batch=1,
            start_pos=self.rows, rope_theta=5e5,
            weight_dtype=self.weight_dtype, rms_eps=self.rms_eps,
            softcap=self.softcap, gated=self.gated, ffn_act=self.ffn_act, seed=self.seed)

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


STACK_CONFIGS: Dict[str, StackConfig] = {
    # 2 layers, hidden 256, 4/2 heads of 64, FFN 704, fp32 weights, 8 tokens.
    "tiny": StackConfig("tiny", 2, 256, 4, 2, 64, 704, batch=8, start_pos=0,
                        rope_theta=1e4, weight_dtype="fp32"),
    # Llama-3.2-3B shape, 28 layers, 512 new tokens, empty cache.
    "llama3b_pp512": StackConfig("llama3b_pp512", 28, 3072, 24, 8, 128, 8192,
                                 batch=512, start_pos=0, rope_theta=5e5),
    # The same stack with 1536 cached rows per layer.
    "llama3b_prefix1536": StackConfig("llama3b_prefix1536", 28, 3072, 24, 8,
                                      128, 8192, batch=512, start_pos=1536,
                                      rope_theta=5e5),
    # Llama-3-8B shape with q/k/v biases and per-head QK RMSNorm, pp4096.
    "llama8b_pp4096_extras": StackConfig("llama8b_pp4096_extras", 32, 4096, 32,
                                         8, 128, 14336, batch=4096,
                                         start_pos=0, rope_theta=5e5,
                                         qkv_bias=True, qk_norm=True),
}

DECODE_CONFIG = DecodeConfig("decode_hq32_hkv8", d_model=4096, n_heads=32,
                             n_kv_heads=8, head_dim=128, d_ff=14336,
                             rows=32768, softcap=50.0, gated=True)
DECODE_ROWS = (32, 300, 4096, 32768)


# --------------------------------------------------------------------------
# encodings of drawn values


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 22
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = ((c + (((c >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def values(a: np.ndarray) -> np.ndarray:
    """The fp32 values a drawn tensor stands for (decodes bf16 patterns)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


# --------------------------------------------------------------------------
# draws


def _normal(seed: int, stream: int, shape, std: float = 1.0,
            mean: float = 0.0) -> np.ndarray:
    g = np.random.Generator(np.random.Philox(key=[seed, stream]))
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def _layer_tensor(cfg: StackConfig, layer: int, name: str, shape) -> np.ndarray:
    stream = (layer + 1) * 32 + _SLOTS[name]
    if name in ("g_attn", "g_ffn", "q_norm", "k_norm", "g_post_attn", "g_post_ffn"):
        return _normal(cfg.seed, stream, shape, 0.02, 1.0)
    a = _normal(cfg.seed, stream, shape, 0.02)
    if name in MATRICES and cfg.weight_dtype == "bf16":
        return to_bf16_bits(a)
    return a


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def layer_weights(cfg: StackConfig, layer: int) -> Dict[str, np.ndarray]:
    """One layer's tensors (matrices as bf16 bit patterns in bf16 configs)."""
    shapes = cfg.shapes()
    with ThreadPoolExecutor(_threads()) as ex:
        futs = {n: ex.submit(_layer_tensor, cfg, layer, n, s) for n, s in shapes.items()}
        return {n: f.result() for n, f in futs.items()}


def hidden_rows(cfg: StackConfig) -> np.ndarray:
    return _normal(cfg.seed, _HIDDEN_STREAM, (cfg.batch, cfg.d_model))


def prefix_rows(cfg: StackConfig, layer: int):
    """(K, V) prefix rows of one layer, ``[start_pos, kv_width]`` fp32 each."""
    shape = (cfg.start_pos, cfg.kv_width)
    base = (layer + 1) * 32
    return (_normal(cfg.seed, base + _SLOTS["prefix_k"], shape),
            _normal(cfg.seed, base + _SLOTS["prefix_v"], shape))


@dataclasses.dataclass
class StackInputs:
    cfg: StackConfig
    layers: List[Dict[str, np.ndarray]]
    hidden: np.ndarray
    prefix_k: List[np.ndarray]
    prefix_v: List[np.ndarray]


def stack_inputs(cfg: StackConfig, n_layers: Optional[int] = None) -> StackInputs:
    """All inputs of a prefill call: weights of the first ``n_layers``
    layers (default: all), the hidden batch and the per-layer prefixes."""
    n = cfg.n_layers if n_layers is None else n_layers
    layers = [layer_weights(cfg, l) for l in range(n)]
    pk, pv = zip(*[prefix_rows(cfg, l) for l in range(n)]) if n else ((), ())
    return StackInputs(cfg, layers, hidden_rows(cfg), list(pk), list(pv))


def decode_inputs(cfg: DecodeConfig) -> Dict[str, np.ndarray]:
    """Inputs of one decode attention layer: the host cache's ``rows`` K/V
    rows, this token's q/k/v (already rotated) and gate, the residual row,
    and the layer's weights."""
    s, b = cfg.seed, _DECODE_STREAM_BASE
    out = {
        "cache_k": _normal(s, b + 0, (cfg.rows, cfg.kv_width)),
        "cache_v": _normal(s, b + 1, (cfg.rows, cfg.kv_width)),
        "q": _normal(s, b + 2, (cfg.q_width,)),
        "k": _normal(s, b + 3, (cfg.kv_width,)),
        "v": _normal(s, b + 4, (cfg.kv_width,)),
        "gate": _normal(s, b + 5, (cfg.q_width,)),
        "residual": _normal(s, b + 6, (cfg.d_model,)),
    }
    out["weights"] = layer_weights(cfg.stack_view(), 0)
    return out

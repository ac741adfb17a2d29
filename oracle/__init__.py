"""CPU oracle for the resident dense prefill stack and the decode attention
layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports, links or calls anything here, and nothing here calls the GPU
library.

Plain float64 numpy, one step after another, in the order the pages give:

* "frink-models 0.29.0 src/decoder/cuda_prefill.rs": the resident prefill
  stack (module doc: hidden goes up once, every step between the seven
  matmuls of a layer runs on the device, each layer's K/V rows come back;
  ``cuda_prefill_layer``: the layer descriptor -- pre-attention and pre-FFN
  RMS norms with one epsilon, q/k/v/o/gate/up/down projections, optional
  q/k/v biases and per-head Q/K norms, RoPE (theta, frequency factors,
  rotated width, Norm/Neox pairing, attention factor), and the attention
  parameters -- head counts, 1/sqrt(head_dim) scale, optional logit
  softcap, the cached prefix and ``start_pos``).
* "frink-models 0.38.0 src/decoder/device_attention.rs": the single-token
  attention layer against the cache's device mirror (``device_attention_
  layer``: attention, output gate, ``wo``, residual, FFN norm, FFN,
  residual, with q/k/v given already rotated and the gate being the half
  split off a double-width ``wq``).
* "frink-models 0.49.0 src/fused_layer.rs": module doc, the layer is
  ``x + ffn(rms_norm(x + branch))`` with one dense SwiGLU expert and a plain
  weighted RMS norm.

The pages do not print the kernels' arithmetic, so each step is the
textbook definition of that step of a pre-norm Llama layer; every point the
pages leave open is a stated reading:

* RMSNorm is ``x / sqrt(mean(x^2) + eps) * g`` (epsilon inside the root,
  gain multiplied as is).
* Query head ``h`` reads KV head ``h // (n_heads / n_kv_heads)``.
* A K/V row is token-major, ``[n_kv_heads][head_dim]`` within the row.
* Order inside the projection step: bias, then per-head RMS norm, then
  RoPE at position ``start_pos + b``, then the attention factor on the
  rotated channels.
* Neox RoPE pairs channel ``i`` with ``i + rot_dim/2``; Norm pairs ``2i``
  with ``2i+1``; the angle of pair ``i`` at position ``p`` is
  ``p * theta^(-2i/rot_dim) / freq_factors[i]``.
* Scores are ``q.k / sqrt(head_dim)``, then ``c*tanh(s/c)`` when a softcap
  ``c`` is set; token ``b`` sees keys ``0 .. start_pos+b`` inclusive; exact
  max-subtracted softmax.
* The output gate multiplies the attention output element-wise by
  ``sigmoid(gate)``; a gated ``wq`` is ``[q rows ; gate rows]``.
* SwiGLU is ``silu(h Wg^T) * (h Wu^T)`` with ``silu(z) = z / (1 + e^-z)``;
  the GELU-gated FFN puts the exact GELU ``z * Phi(z)`` (normal CDF, erf
  form) in place of silu.
* A sliding window ``W`` lets the token at position ``p`` see keys
  ``p-W+1 .. p`` (its own key and the ``W-1`` before it).
* A sandwich-norm layer RMS-normalises each branch output with its own gain
  (``g_post_attn``, ``g_post_ffn``, the same epsilon) before the residual
  add: ``x1 = x + rms_norm(attn) * g_post_attn``, ``out = x1 +
  rms_norm(ffn) * g_post_ffn``.
* The stack returns the last layer's residual stream, with no final norm.
* The decode layer attends over the cached rows plus its own new row.

Weights are ``[out, in]`` row-major and ``y = W x``.
"""
from __future__ import annotations

from typing import Iterable, List, Mapping, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "rms_norm", "rope_angles", "apply_rope", "causal_gqa_attention", "silu", "gelu",
    "swiglu_ffn", "project_qkv", "dense_layer", "prefill_dense_stack",
    "attn_layer", "decode_layer", "kv_head_of",
]

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """Weighted RMS norm over the last axis.

    fused_layer.rs (0.49.0), "What it refuses" and ``LayerFfnParts::
    for_layer``: the pre-FFN norm must be a plain weighted RMS norm;
    cuda_prefill.rs (0.29.0), ``try_cuda_prefill_dense_stack``: one epsilon
    for the whole layer.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gain)


def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """GQA head map (reading: contiguous groups).

    device_attention.rs (0.38.0), ``device_attention_layer``: the layer's
    shape is ``Gqa { n_heads, n_kv_heads }``.
    """
    return h // (n_heads // n_kv_heads)


def rope_angles(positions, rot_dim: int, theta: float,
                freq_factors=None) -> np.ndarray:
    """Angles ``[len(positions), rot_dim/2]`` of each rotated pair.

    cuda_prefill.rs (0.29.0), ``cuda_prefill_layer``: the layer's RoPE
    carries theta, optional per-pair frequency factors and the rotated
    width (default: the head width).
    """
    i = np.arange(rot_dim // 2, dtype=F64)
    inv_freq = theta ** (-2.0 * i / rot_dim)
    if freq_factors is not None:
        inv_freq = inv_freq / _f64(freq_factors)
    return _f64(positions)[:, None] * inv_freq[None, :]


def apply_rope(x, positions, theta: float, layout: str = "neox",
               rot_dim: Optional[int] = None, freq_factors=None,
               mscale: float = 1.0) -> np.ndarray:
    """Rotate ``x [T, H, hd]`` by the angles of ``positions [T]``.

    cuda_prefill.rs (0.29.0), ``cuda_prefill_layer``: Norm (adjacent pairs)
    or Neox (half split) layout; the attention factor scales the rotated
    channels of Q and K.
    """
    x = _f64(x).copy()
    hd = x.shape[-1]
    rd = hd if rot_dim is None else rot_dim
    ang = rope_angles(positions, rd, theta, freq_factors)[:, None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    if layout == "neox":
        a, b = x[..., : rd // 2].copy(), x[..., rd // 2: rd].copy()
        x[..., : rd // 2] = a * cos - b * sin
        x[..., rd // 2: rd] = a * sin + b * cos
    elif layout == "norm":
        a, b = x[..., 0:rd:2].copy(), x[..., 1:rd:2].copy()
        x[..., 0:rd:2] = a * cos - b * sin
        x[..., 1:rd:2] = a * sin + b * cos
    else:
        raise ValueError(f"unknown RoPE layout {layout!r}")
    if mscale != 1.0:
        x[..., :rd] *= mscale
    return x


def causal_gqa_attention(q, k_all, v_all, start_pos: int, softcap: float = 0.0,
                         gate=None, window: int = 0) -> np.ndarray:
    """Causal GQA attention of ``B`` new tokens over ``start_pos`` cached
    rows followed by the new rows.

    ``q [B, Hq, hd]``; ``k_all, v_all [start_pos + B, Hkv, hd]`` (key ``j``
    is cached row ``j`` for ``j < start_pos`` and new row ``j - start_pos``
    after); ``gate [B, Hq, hd]`` or None.  Returns ``o [B, Hq, hd]``.

    cuda_prefill.rs (0.29.0), ``cuda_prefill_layer``: the attention
    parameters -- head counts, scale 1/sqrt(head_dim), optional softcap, the
    cache prefix, ``start_pos``, the sliding ``window``; device_attention.rs
    (0.38.0), ``device_attention_layer``: the gate is applied to the
    attention output.
    """
    q, k_all, v_all = _f64(q), _f64(k_all), _f64(v_all)
    B, Hq, hd = q.shape
    T, Hkv, _ = k_all.shape
    assert T == start_pos + B
    scale = 1.0 / np.sqrt(hd)
    # key j is visible to token b iff j <= start_pos + b
    pos = (start_pos + np.arange(B))[:, None]
    visible = np.arange(T)[None, :] <= pos
    if window:
        visible &= np.arange(T)[None, :] > pos - window
    o = np.empty((B, Hq, hd), F64)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        s = (q[:, h, :] @ k_all[:, g, :].T) * scale
        if softcap:
            s = softcap * np.tanh(s / softcap)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v_all[:, g, :]
    if gate is not None:
        o = o * (1.0 / (1.0 + np.exp(-_f64(gate))))
    return o


def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def gelu(z) -> np.ndarray:
    """Exact GELU, ``z * Phi(z)`` with the standard normal CDF."""
    from scipy.special import erf
    z = _f64(z)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def swiglu_ffn(h2, wg, wu, wd, act: str = "swiglu") -> np.ndarray:
    """``(act(h2 Wg^T) * (h2 Wu^T)) Wd^T`` with ``act`` silu (SwiGLU) or
    GELU (the GELU-gated FFN).

    cuda_prefill.rs (0.29.0), ``try_cuda_prefill_dense_stack``: the fused
    body's activation is SwiGLU, the other gated activation is GELU;
    fused_layer.rs (0.49.0): one dense expert's gate, up and down.
    """
    h2 = _f64(h2)
    g = h2 @ _f64(wg).T
    a = gelu(g) if act == "geglu" else silu(g)
    return (a * (h2 @ _f64(wu).T)) @ _f64(wd).T


def project_qkv(h, w: Mapping[str, np.ndarray], spec, positions):
    """Q/K/V (and gate) of normed rows ``h [T, d]`` at ``positions [T]``.

    Returns ``q [T, Hq, hd]``, ``gate [T, Hq, hd]`` or None,
    ``k, v [T, Hkv, hd]``; q and k are biased, QK-normed and rotated, v is
    biased.  cuda_prefill.rs (0.29.0), ``cuda_prefill_layer``: separate q, k,
    v projections, the optional extras (biases, Q/K norms) and the RoPE
    description; device_attention.rs (0.38.0): the gate is the second half
    of a double-width ``wq``.
    """
    h = _f64(h)
    T = h.shape[0]
    Hq, Hkv, hd = spec.n_heads, spec.n_kv_heads, spec.head_dim
    qg = h @ _f64(w["wq"]).T
    q, gate = qg[:, : Hq * hd], None
    if getattr(spec, "gated", False):
        gate = qg[:, Hq * hd:].reshape(T, Hq, hd)
    k = h @ _f64(w["wk"]).T
    v = h @ _f64(w["wv"]).T
    if getattr(spec, "qkv_bias", False):
        q, k, v = q + _f64(w["bq"]), k + _f64(w["bk"]), v + _f64(w["bv"])
    q, k, v = q.reshape(T, Hq, hd), k.reshape(T, Hkv, hd), v.reshape(T, Hkv, hd)
    if getattr(spec, "qk_norm", False):
        q = rms_norm(q, w["q_norm"], spec.rms_eps)
        k = rms_norm(k, w["k_norm"], spec.rms_eps)
    if getattr(spec, "rope_theta", None):
        rope = dict(layout=getattr(spec, "rope_layout", "neox"),
                    rot_dim=getattr(spec, "rope_rot_dim", 0) or None,
                    freq_factors=getattr(spec, "rope_freq_factors", None),
                    mscale=getattr(spec, "rope_mscale", 1.0))
        q = apply_rope(q, positions, spec.rope_theta, **rope)
        k = apply_rope(k, positions, spec.rope_theta, **rope)
    return q, gate, k, v


def dense_layer(x, w: Mapping[str, np.ndarray], spec, start_pos: int,
                prefix_k=None, prefix_v=None):
    """One pre-norm dense layer over ``B`` new tokens.

    ``x [B, d]``; ``prefix_k, prefix_v [start_pos, Hkv*hd]`` are the cached
    rows, used as they are (already rotated).  Returns ``(x_out, k_rows,
    v_rows)`` with ``k_rows, v_rows [B, Hkv*hd]`` -- exactly the rows the
    caller pushes into its cache.

    fused_layer.rs (0.49.0), module doc: ``x + ffn(rms_norm(x + branch))``;
    cuda_prefill.rs (0.29.0), ``try_cuda_prefill_dense_stack``: each layer's
    K/V rows come back, one ``kv_width`` row per token; ``cuda_prefill_
    layer``: the optional post-attention and post-FFN norms (present when
    ``w`` holds ``g_post_attn`` / ``g_post_ffn``).
    """
    x = _f64(x)
    B = x.shape[0]
    Hkv, hd = spec.n_kv_heads, spec.head_dim
    positions = start_pos + np.arange(B)
    h = rms_norm(x, w["g_attn"], spec.rms_eps)
    q, gate, k, v = project_qkv(h, w, spec, positions)
    if start_pos:
        k_all = np.concatenate([_f64(prefix_k).reshape(start_pos, Hkv, hd), k])
        v_all = np.concatenate([_f64(prefix_v).reshape(start_pos, Hkv, hd), v])
    else:
        k_all, v_all = k, v
    o = causal_gqa_attention(q, k_all, v_all, start_pos,
                             getattr(spec, "softcap", 0.0), gate,
                             getattr(spec, "window", 0))
    attn = o.reshape(B, -1) @ _f64(w["wo"]).T
    if "g_post_attn" in w:
        attn = rms_norm(attn, w["g_post_attn"], spec.rms_eps)
    x1 = x + attn
    h2 = rms_norm(x1, w["g_ffn"], spec.rms_eps)
    ffn = swiglu_ffn(h2, w["wg"], w["wu"], w["wd"], getattr(spec, "ffn_act", "swiglu"))
    if "g_post_ffn" in w:
        ffn = rms_norm(ffn, w["g_post_ffn"], spec.rms_eps)
    x2 = x1 + ffn
    return x2, k.reshape(B, Hkv * hd), v.reshape(B, Hkv * hd)


def prefill_dense_stack(hidden, layers: Iterable[Mapping[str, np.ndarray]],
                        spec, start_pos: int = 0,
                        prefix_k: Optional[Sequence] = None,
                        prefix_v: Optional[Sequence] = None
                        ) -> Tuple[np.ndarray, List[np.ndarray], List[np.ndarray]]:
    """A run of consecutive dense layers; returns ``(hidden_out, k_rows[l],
    v_rows[l])``.

    cuda_prefill.rs (0.29.0), module doc and ``try_cuda_prefill_dense_stack``:
    the hidden batch enters once and leaves after the last layer of the run;
    every layer attends over its own cache's prefix.  ``layers`` may be any
    iterable (a generator keeps one layer's weights alive at a time).
    """
    x = _f64(hidden)
    ks, vs = [], []
    for l, w in enumerate(layers):
        pk = prefix_k[l] if start_pos else None
        pv = prefix_v[l] if start_pos else None
        x, k, v = dense_layer(x, w, spec, start_pos, pk, pv)
        ks.append(k)
        vs.append(v)
    return x, ks, vs


def attn_layer(q, k, v, gate, cache_k, cache_v, rows: int,
               w: Mapping[str, np.ndarray], spec, residual) -> np.ndarray:
    """One token's attention layer against the cache: attend over the
    ``rows`` cached rows plus this token's own ``k``/``v``, gate, ``wo``,
    residual, FFN norm, SwiGLU FFN, residual.

    ``q, gate [Hq*hd]`` (gate may be None), ``k, v [Hkv*hd]`` already rotated
    and QK-normed; ``cache_k, cache_v [>= rows, Hkv*hd]``.

    device_attention.rs (0.38.0), ``device_attention_layer`` (the one
    submission) and ``ensure_attn_mirror`` (the mirror must hold exactly the
    cache's rows; the launch needs room for one more row).
    """
    Hq, Hkv, hd = spec.n_heads, spec.n_kv_heads, spec.head_dim
    k_all = np.concatenate([_f64(cache_k)[:rows], _f64(k)[None]]).reshape(rows + 1, Hkv, hd)
    v_all = np.concatenate([_f64(cache_v)[:rows], _f64(v)[None]]).reshape(rows + 1, Hkv, hd)
    g = None if gate is None else _f64(gate).reshape(1, Hq, hd)
    o = causal_gqa_attention(_f64(q).reshape(1, Hq, hd), k_all, v_all, rows,
                             getattr(spec, "softcap", 0.0), g)
    x1 = _f64(residual) + _f64(w["wo"]) @ o.reshape(-1)
    h2 = rms_norm(x1, w["g_ffn"], spec.rms_eps)
    return x1 + swiglu_ffn(h2[None], w["wg"], w["wu"], w["wd"],
                           getattr(spec, "ffn_act", "swiglu"))[0]


def decode_layer(x, w: Mapping[str, np.ndarray], spec, cache_k, cache_v, rows: int):
    """One token's whole layer at position ``rows``: attention norm, the
    q/k/v(/gate) projection with its extras and RoPE, then ``attn_layer``
    over the ``rows`` cached rows plus this token's own.  Returns ``(out,
    k_row, v_row)``; the rows are the ones the caller pushes into its cache.

    fused_layer.rs (0.49.0), module doc ("Why": one submission a layer) and
    device_attention.rs (0.38.0), ``device_attention_layer`` (q/k/v
    post-RoPE and post-QK-norm feed the device attention); the head follows
    cuda_prefill.rs (0.29.0), ``cuda_prefill_layer``.
    """
    x = _f64(x)
    h = rms_norm(x[None], w["g_attn"], spec.rms_eps)
    q, gate, k, v = project_qkv(h, w, spec, [rows])
    out = attn_layer(q.reshape(-1), k.reshape(-1), v.reshape(-1),
                     None if gate is None else gate.reshape(-1), cache_k, cache_v, rows, w,
                     spec, x)
    return out, k.reshape(-1), v.reshape(-1)

"""Resident dense decoder-layer stack for AMD MI355X (gfx950).

Python binding of libddl.so: every ``ddl_*`` function here has the name and
the arguments of the C entry point in include/ddl.h and only marshals them
(torch tensors -> device pointers, the current torch stream -> hipStream_t).
All arithmetic runs in the library's HIP kernels; importing this package on
a machine without the built library raises.

PyTorch provides device memory and streams.  ``pack_layer_from_host`` and
``new_*`` are allocation conveniences for callers that hold host arrays.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int, c_void_p
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _native as N
from ._native import (DDL_K_ATTN_PREFILL, DDL_K_DECODE_ATTN, DDL_K_DECODE_HEAD, DDL_K_GEMM_DOWN,
                      DDL_K_GEMM_GATE_UP, DDL_K_GEMM_QKV, DDL_K_GEMM_WO, DDL_K_GEMV_DOWN,
                      DDL_K_GEMV_GATE_UP, DDL_K_GEMV_QKV, DDL_K_GEMV_WO, DDL_K_QKV_POST,
                      DDL_K_RMSNORM)
from ._native import (DDL_ACT_GELU, DDL_ACT_SWIGLU, DDL_DECLINED, DDL_DTYPE_BF16,
                      DDL_DTYPE_F32, DDL_ERR_DEVICE, DDL_ERR_INJECTED, DDL_ERR_INVALID,
                      DDL_ERR_WORKSPACE, DDL_NOALLOC_SCRATCH_BYTES, DDL_ROPE_NEOX,
                      DDL_ATTN_AUTO, DDL_ATTN_ONE_HEAD, DDL_ATTN_SHARED,
                      DDL_ROPE_NORM, CtxOpts, LayerDesc, LayerWeights)

__all__ = [
    "ddl_ctx_create", "ddl_ctx_destroy", "ddl_layer_supported", "ddl_layer_blob_bytes",
    "ddl_layer_pack", "ddl_layer_destroy", "ddl_workspace_bytes", "ddl_prefill_dense_stack",
    "ddl_mirror_bytes", "ddl_mirror_init", "ddl_mirror_upload", "ddl_mirror_seq_len",
    "ddl_mirror_capacity", "ddl_mirror_invalidate", "ddl_mirror_plan_capacity",
    "ddl_mirror_destroy", "ddl_attn_workspace_bytes", "ddl_attn_layer", "ddl_attn_layer_noalloc",
    "ddl_decode_layer", "ddl_decode_graph_create", "ddl_decode_graph_launch",
    "ddl_decode_graph_destroy", "DecodeGraph",
    "ddl_last_error",
    "ddl_probe_enable", "ddl_probe_read",
    "layer_desc", "pack_layer_from_host", "Ctx", "Layer", "Mirror", "LayerDesc",
]


def _lib():
    return N.lib()


_lib()   # no library, no package: there is no fallback path


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def ddl_last_error() -> str:
    return _lib().ddl_last_error().decode()


def ddl_probe_enable(ctx: "Ctx", kind: int, max_launches: int) -> int:
    rc = _lib().ddl_probe_enable(ctx.handle, kind, max_launches)
    if rc < 0:
        raise RuntimeError(f"ddl_probe_enable: {rc} {ddl_last_error()}")
    return rc


def ddl_probe_read(ctx: "Ctx", cap: int = 4096) -> List[float]:
    """Durations (ms) of the launches bracketed since ddl_probe_enable."""
    buf = (ctypes.c_float * cap)()
    n = _lib().ddl_probe_read(ctx.handle, buf, cap)
    if n < 0:
        raise RuntimeError(f"ddl_probe_read: {n} {ddl_last_error()}")
    return [buf[i] for i in range(min(n, cap))]


# ---- context ------------------------------------------------------------------


class Ctx:
    def __init__(self, handle: int):
        self.handle = handle

    def __del__(self):
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "handle", None) and ddl_ctx_destroy is not None:
            ddl_ctx_destroy(self)


def ddl_ctx_create(min_batch: int = 4, fault_after_admission: bool = False,
                   attn_form: int = 0) -> Ctx:
    """attn_form: DDL_ATTN_AUTO, DDL_ATTN_ONE_HEAD or DDL_ATTN_SHARED."""
    opts = CtxOpts(min_batch, int(fault_after_admission), int(attn_form))
    h = _lib().ddl_ctx_create(byref(opts))
    if not h:
        raise MemoryError("ddl_ctx_create")
    return Ctx(h)


def ddl_ctx_destroy(ctx: Ctx) -> None:
    if ctx.handle:
        _lib().ddl_ctx_destroy(ctx.handle)
        ctx.handle = None


# ---- layers -------------------------------------------------------------------


def layer_desc(d_model: int, n_heads: int, n_kv_heads: int, head_dim: int, d_ff: int,
               rms_eps: float = 1e-5, rope_theta: Optional[float] = 1e4,
               softcap: float = 0.0, gated: bool = False, qkv_bias: bool = False,
               qk_norm: bool = False, **extra) -> LayerDesc:
    """A ddl_layer_desc; ``extra`` sets any other field by its C name."""
    d = LayerDesc()
    d.d_model, d.n_heads, d.n_kv_heads, d.head_dim = d_model, n_heads, n_kv_heads, head_dim
    d.v_head_dim, d.d_ff = head_dim, d_ff
    d.rms_eps = d.post_norm_eps = rms_eps
    d.act = DDL_ACT_SWIGLU
    d.rope_enabled = int(bool(rope_theta))
    d.rope_theta = float(rope_theta or 0.0)
    d.rope_layout = DDL_ROPE_NEOX
    d.rope_rot_dim = 0
    d.rope_mscale = 1.0
    d.rope_freq_factors = None
    d.attn_softcap = softcap
    d.gated, d.has_qkv_bias, d.has_qk_norm = int(gated), int(qkv_bias), int(qk_norm)
    for k, v in extra.items():
        if k == "rope_freq_factors" and v is not None:
            # a host float array the descriptor points at; kept alive with it
            arr = (ctypes.c_float * len(v))(*[float(x) for x in v])
            d._freq_keep = arr
            v = ctypes.cast(arr, c_void_p)
        setattr(d, k, v)
    return d


class Layer:
    """A packed layer: the library handle plus the device blob it borrows."""

    def __init__(self, handle: int, blob: torch.Tensor, desc: LayerDesc):
        self.handle, self.blob, self.desc = handle, blob, desc

    def __del__(self):
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "handle", None) and ddl_layer_destroy is not None:
            ddl_layer_destroy(self)


def ddl_layer_supported(desc: LayerDesc) -> bool:
    return bool(_lib().ddl_layer_supported(byref(desc)))


def ddl_layer_blob_bytes(desc: LayerDesc) -> int:
    return int(_lib().ddl_layer_blob_bytes(byref(desc)))


_WEIGHT_KEYS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "g_attn", "g_ffn", "bq", "bk", "bv",
                "q_norm", "k_norm", "g_post_attn", "g_post_ffn")


def ddl_layer_pack(ctx: Ctx, desc: LayerDesc, weights: Dict[str, torch.Tensor], dtype: int,
                   blob: torch.Tensor, stream=None) -> Optional[Layer]:
    """Packs device tensors ``weights`` into ``blob``; None when declined."""
    w = LayerWeights()
    w.dtype = dtype
    for k in _WEIGHT_KEYS:
        setattr(w, k, _ptr(weights.get(k)))
    out = c_void_p()
    rc = _lib().ddl_layer_pack(ctx.handle, byref(desc), byref(w), blob.data_ptr(),
                               blob.numel() * blob.element_size(), _stream(stream), byref(out))
    if rc == DDL_DECLINED:
        return None
    if rc < 0:
        raise RuntimeError(f"ddl_layer_pack: {rc} {ddl_last_error()}")
    return Layer(out.value, blob, desc)


def ddl_layer_destroy(layer: Layer) -> None:
    if layer.handle:
        _lib().ddl_layer_destroy(layer.handle)
        layer.handle = None


def pack_layer_from_host(ctx: Ctx, desc: LayerDesc, host: Dict[str, np.ndarray],
                         device="cuda") -> Optional[Layer]:
    """Uploads host weights (matrices as fp32, or bf16 bit patterns in uint16)
    and packs them; the staging copies are released after the pack ran."""
    mats = [host[k] for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]
    dtype = DDL_DTYPE_BF16 if mats[0].dtype == np.uint16 else DDL_DTYPE_F32
    staged = {}
    for k, a in host.items():
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a.astype(np.float32))
        staged[k] = t.to(device, non_blocking=False)
    blob = torch.empty(ddl_layer_blob_bytes(desc), dtype=torch.uint8, device=device)
    layer = ddl_layer_pack(ctx, desc, staged, dtype, blob)
    torch.cuda.current_stream().synchronize()
    del staged
    return layer


def ddl_workspace_bytes(layers: Sequence[Layer], max_batch: int, max_start_pos: int) -> int:
    arr = (c_void_p * len(layers))(*[l.handle for l in layers])
    return int(_lib().ddl_workspace_bytes(arr, len(layers), max_batch, max_start_pos))


def ddl_prefill_dense_stack(ctx: Ctx, hidden: torch.Tensor, layers: Sequence[Layer],
                            start_pos: int, prefix_k: Optional[Sequence[torch.Tensor]],
                            prefix_v: Optional[Sequence[torch.Tensor]],
                            prefix_rows: Sequence[int], hidden_out: torch.Tensor,
                            k_rows: Sequence[torch.Tensor], v_rows: Sequence[torch.Tensor],
                            workspace: torch.Tensor, stream=None) -> int:
    """Returns run_len (> 0), 0 when declined; raises on errors (< 0)."""
    n = len(layers)
    arr = lambda xs: (c_void_p * n)(*[None if x is None else _ptr(x) for x in xs])
    pk = arr(prefix_k) if prefix_k is not None else None
    pv = arr(prefix_v) if prefix_v is not None else None
    rows = (c_int * n)(*prefix_rows)
    rc = _lib().ddl_prefill_dense_stack(
        ctx.handle, hidden.data_ptr(), (c_void_p * n)(*[l.handle for l in layers]), n,
        hidden.shape[0], start_pos, pk, pv, rows, hidden_out.data_ptr(), arr(k_rows),
        arr(v_rows), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_prefill_dense_stack: {rc} {ddl_last_error()}")
    return rc


# ---- mirror -------------------------------------------------------------------


class Mirror:
    def __init__(self, handle: int, buf: torch.Tensor):
        self.handle, self.buf = handle, buf

    def __del__(self):
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "handle", None) and ddl_mirror_destroy is not None:
            ddl_mirror_destroy(self)


def ddl_mirror_bytes(n_kv_heads: int, head_dim: int, capacity: int) -> int:
    return int(_lib().ddl_mirror_bytes(n_kv_heads, head_dim, capacity))


def ddl_mirror_init(buf: torch.Tensor, n_kv_heads: int, head_dim: int, capacity: int) -> Mirror:
    out = c_void_p()
    rc = _lib().ddl_mirror_init(byref(out), buf.data_ptr(), buf.numel() * buf.element_size(),
                                n_kv_heads, head_dim, capacity)
    if rc != 1:
        raise RuntimeError(f"ddl_mirror_init: {rc} {ddl_last_error()}")
    return Mirror(out.value, buf)


def ddl_mirror_upload(m: Mirror, k, v, rows: int, stream=None) -> int:
    """k, v: torch tensors (host or device) of [>= rows][kv_width] fp32."""
    rc = _lib().ddl_mirror_upload(m.handle, _ptr(k), _ptr(v), rows, _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_mirror_upload: {rc} {ddl_last_error()}")
    return rc


def ddl_mirror_seq_len(m: Mirror) -> int:
    return int(_lib().ddl_mirror_seq_len(m.handle))


def ddl_mirror_capacity(m: Mirror) -> int:
    return int(_lib().ddl_mirror_capacity(m.handle))


def ddl_mirror_invalidate(m: Mirror) -> None:
    _lib().ddl_mirror_invalidate(m.handle)


def ddl_mirror_plan_capacity(rows: int, planned: int = 0) -> int:
    return int(_lib().ddl_mirror_plan_capacity(rows, planned))


def ddl_mirror_destroy(m: Mirror) -> None:
    if m.handle:
        _lib().ddl_mirror_destroy(m.handle)
        m.handle = None


def ddl_attn_workspace_bytes(layer: Layer, capacity: int) -> int:
    return int(_lib().ddl_attn_workspace_bytes(layer.handle, capacity))


def ddl_attn_layer(ctx: Ctx, mirror: Mirror, host_rows: int, q: torch.Tensor, k: torch.Tensor,
                   v: torch.Tensor, gate: Optional[torch.Tensor], n_heads: int, softcap: float,
                   layer: Layer, residual: torch.Tensor, out: torch.Tensor,
                   workspace: torch.Tensor, stream=None) -> int:
    """Returns 1 (served), 0 (declined); raises on errors (< 0)."""
    rc = _lib().ddl_attn_layer(ctx.handle, mirror.handle, host_rows, q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), _ptr(gate), n_heads, float(softcap), layer.handle,
                               residual.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_attn_layer: {rc} {ddl_last_error()}")
    return rc


def ddl_attn_layer_noalloc(ctx: Ctx, mirror: Mirror, host_rows: int, q: torch.Tensor,
                           k: torch.Tensor, v: torch.Tensor, gate: Optional[torch.Tensor],
                           n_heads: int, softcap: float, layer: Layer, residual: torch.Tensor,
                           out: torch.Tensor, stream=None) -> int:
    """ddl_attn_layer with the library's fixed device scratch instead of a
    workspace.  Returns 1 (served), 0 (declined); raises on errors (< 0)."""
    rc = _lib().ddl_attn_layer_noalloc(ctx.handle, mirror.handle, host_rows, q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), _ptr(gate), n_heads,
                                       float(softcap), layer.handle, residual.data_ptr(),
                                       out.data_ptr(), _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_attn_layer_noalloc: {rc} {ddl_last_error()}")
    return rc


def ddl_decode_layer(ctx: Ctx, mirror: Mirror, host_rows: int, hidden: torch.Tensor, layer: Layer,
                     out: torch.Tensor, k_row: torch.Tensor, v_row: torch.Tensor,
                     workspace: torch.Tensor, stream=None) -> int:
    """Returns 1 (served), 0 (declined); raises on errors (< 0)."""
    rc = _lib().ddl_decode_layer(ctx.handle, mirror.handle, host_rows, hidden.data_ptr(),
                                 layer.handle, out.data_ptr(), k_row.data_ptr(), v_row.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_decode_layer: {rc} {ddl_last_error()}")
    return rc


class DecodeGraph:
    """A captured decode step; keeps the buffers it is bound to alive."""

    def __init__(self, handle: int, keep):
        self.handle, self._keep = handle, keep

    def __del__(self):
        if getattr(self, "handle", None) and ddl_decode_graph_destroy is not None:
            ddl_decode_graph_destroy(self)


def ddl_decode_graph_create(ctx: Ctx, mirror: Mirror, layer: Layer, hidden: torch.Tensor,
                            out: torch.Tensor, k_row: torch.Tensor, v_row: torch.Tensor,
                            workspace: torch.Tensor) -> Optional[DecodeGraph]:
    """Captures one ddl_decode_layer step bound to these buffers; None when
    declined; raises on errors."""
    g = c_void_p()
    rc = _lib().ddl_decode_graph_create(ctx.handle, mirror.handle, layer.handle,
                                        hidden.data_ptr(), out.data_ptr(), k_row.data_ptr(),
                                        v_row.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), byref(g))
    if rc < 0:
        raise RuntimeError(f"ddl_decode_graph_create: {rc} {ddl_last_error()}")
    if rc == 0:
        return None
    return DecodeGraph(g.value, (ctx, mirror, layer, hidden, out, k_row, v_row, workspace))


def ddl_decode_graph_launch(ctx: Ctx, graph: DecodeGraph, host_rows: int, stream=None) -> int:
    """Returns 1 (served), 0 (declined); raises on errors (< 0)."""
    rc = _lib().ddl_decode_graph_launch(ctx.handle, graph.handle, host_rows, _stream(stream))
    if rc < 0:
        raise RuntimeError(f"ddl_decode_graph_launch: {rc} {ddl_last_error()}")
    return rc


def ddl_decode_graph_destroy(graph: DecodeGraph) -> None:
    if graph.handle:
        _lib().ddl_decode_graph_destroy(graph.handle)
        graph.handle = None


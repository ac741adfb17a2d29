"""Allocation helpers for callers holding host arrays: pack a run of layers
from host weights and allocate the outputs and workspace of a prefill call.
No arithmetic here -- the kernels do all of it."""
from __future__ import annotations

from typing import Iterable, List, Mapping, Optional, Sequence

import numpy as np
import torch

from . import (DDL_ACT_GELU, DDL_ACT_SWIGLU, DDL_ROPE_NEOX, DDL_ROPE_NORM, Ctx, Layer,
               ddl_prefill_dense_stack, ddl_workspace_bytes, layer_desc, pack_layer_from_host)


def desc_for(cfg):
    """ddl_layer_desc of a layer shaped like ``cfg`` (any object with the
    fields d_model, n_heads, n_kv_heads, head_dim, d_ff, rms_eps and,
    optionally, rope_theta, rope_layout, rope_rot_dim, rope_mscale,
    rope_freq_factors, softcap, gated, qkv_bias, qk_norm, ffn_act, window,
    post_norms)."""
    layout = {"neox": DDL_ROPE_NEOX, "norm": DDL_ROPE_NORM}[getattr(cfg, "rope_layout", "neox")]
    act = {"swiglu": DDL_ACT_SWIGLU, "geglu": DDL_ACT_GELU}[getattr(cfg, "ffn_act", "swiglu")]
    return layer_desc(cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ff,
                      rms_eps=cfg.rms_eps, rope_theta=getattr(cfg, "rope_theta", None),
                      softcap=getattr(cfg, "softcap", 0.0), gated=getattr(cfg, "gated", False),
                      qkv_bias=getattr(cfg, "qkv_bias", False),
                      qk_norm=getattr(cfg, "qk_norm", False),
                      rope_layout=layout, rope_rot_dim=getattr(cfg, "rope_rot_dim", 0),
                      rope_mscale=getattr(cfg, "rope_mscale", 1.0),
                      rope_freq_factors=getattr(cfg, "rope_freq_factors", None),
                      act=act, window=getattr(cfg, "window", 0),
                      has_post_attn_norm=int(getattr(cfg, "post_norms", False)),
                      has_post_ffn_norm=int(getattr(cfg, "post_norms", False)))


class DeviceStack:
    """A run of packed layers plus the buffers of one prefill call."""

    def __init__(self, ctx: Ctx, cfg, host_layers: Iterable[Mapping[str, np.ndarray]],
                 device: str = "cuda"):
        self.ctx, self.cfg, self.device = ctx, cfg, device
        self.desc = desc_for(cfg)
        self.layers: List[Layer] = []
        for w in host_layers:
            layer = pack_layer_from_host(ctx, self.desc, w, device)
            if layer is None:
                raise ValueError("layer declined by ddl_layer_pack")
            self.layers.append(layer)

    def buffers(self, batch: int, start_pos: int = 0):
        kvw = self.cfg.n_kv_heads * self.cfg.head_dim
        n = len(self.layers)
        f32 = dict(dtype=torch.float32, device=self.device)
        return {
            "hidden_out": torch.empty(batch, self.cfg.d_model, **f32),
            "k_rows": [torch.empty(batch, kvw, **f32) for _ in range(n)],
            "v_rows": [torch.empty(batch, kvw, **f32) for _ in range(n)],
            "workspace": torch.empty(ddl_workspace_bytes(self.layers, batch, start_pos),
                                     dtype=torch.uint8, device=self.device),
        }

    def run(self, hidden: torch.Tensor, start_pos: int,
            prefix_k: Optional[Sequence[torch.Tensor]], prefix_v: Optional[Sequence[torch.Tensor]],
            bufs, prefix_rows: Optional[Sequence[int]] = None, stream=None) -> int:
        rows = prefix_rows if prefix_rows is not None else [start_pos] * len(self.layers)
        return ddl_prefill_dense_stack(self.ctx, hidden, self.layers, start_pos, prefix_k, prefix_v,
                                       rows, bufs["hidden_out"], bufs["k_rows"], bufs["v_rows"],
                                       bufs["workspace"], stream)

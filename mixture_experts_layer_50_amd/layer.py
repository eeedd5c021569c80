"""Device buffers for one MoE layer and the order of C-ABI calls of a
forward and a backward pass.  Plumbing only: torch allocates device memory,
every step runs in libmoe.so."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

from . import binding as B


def torch_dtype(shape: B.MoEShape):
    return torch.bfloat16 if shape.dtype == B.DTYPES["bf16"] else torch.float32


@dataclass
class LayerBuffers:
    """Every intermediate and gradient buffer of the layer, sized for the
    row capacity R_cap (T*k unless the shape says otherwise)."""
    shape: B.MoEShape
    device: str = "cuda"
    training: bool = True
    gather: bool = False  # FFN reads x through perm (the _gather calls); no Xp buffer
    fused: bool = False   # gathered FFN forward with the combine in its epilogue (implies gather)
    aux_alpha: Optional[float] = None  # router balancing loss weight (softmax top-k gate)
    # gathered backward with the combine backward inside it
    # (moe_combine_ffn_bwd_gather): dYp written only where a kernel reads it,
    # else its rows formed from dY and the gate weights inside the kernels
    # (implies gather)
    dy_form: bool = False
    t: Dict[str, torch.Tensor] = field(default_factory=dict)

    def __post_init__(self):
        if self.fused or self.dy_form:
            self.gather = True
        s, dev = self.shape, self.device
        dt = torch_dtype(s)
        R, T, d, E, k, I, El = s.rows_cap, s.T, s.d, s.E, s.k, s.I, s.E_loc
        f32, i32 = torch.float32, torch.int32

        def e(*shp, dtype=dt):
            return torch.empty(shp, dtype=dtype, device=dev)

        t = self.t
        t["logits"] = e(T, E, dtype=f32)
        t["topk_idx"] = e(T, k, dtype=i32)
        t["topk_w"] = e(T, k, dtype=f32)
        t["offsets"] = e(El + 1, dtype=i32)
        t["perm"] = e(R, dtype=i32)
        t["inv"] = e(T * k, dtype=i32)
        t["xp"] = None if self.gather else e(R, d)
        t["h"] = e(R, 2 * I) if self.training else None
        t["a"] = e(R, I)
        t["yp"] = e(R, d)
        t["y"] = e(T, d)
        for op in ("permute", "route_permute", "ffn_fwd_fused" if self.fused else "ffn_fwd"):
            t["ws_" + op] = self._ws(op)
        if self.aux_alpha is not None:
            t["aux_loss"] = e(1, dtype=f32)
            t["aux_w"] = e(E, dtype=f32)
            t["ws_aux_loss"] = self._ws("aux_loss")
        if self.training:
            t["dyp"] = e(R, d)
            t["dtopk_w"] = e(T, k, dtype=f32)
            t["dxp"] = e(R, d)
            t["dw_gate"] = e(El, d, I)
            t["dw_up"] = e(El, d, I)
            t["dw_down"] = e(El, I, d)
            t["dx"] = e(T, d)
            t["dlogits"] = e(T, E, dtype=f32)
            t["dw_router"] = e(d, E)
            t["dbias"] = e(E, dtype=f32)
            if s.gate == B.GATES["balanced"]:
                # the balanced gate's weights are constants: the router
                # gradients are identically zero, set once here (the backward
                # passes NULL for them, so nothing rewrites them)
                for name in ("dlogits", "dw_router", "dbias"):
                    t[name].zero_()
            for op in ("ffn_bwd", "route_bwd"):
                t["ws_" + op] = self._ws(op)

    def _ws(self, op) -> Optional[torch.Tensor]:
        n = B.workspace_size(self.shape, op)
        return torch.empty(n, dtype=torch.uint8, device=self.device) if n else None

    def __getitem__(self, k):
        return self.t[k]


def forward(shape: B.MoEShape, buf: LayerBuffers, x, w_router, bias, w_gate, w_up, w_down,
            stream=None):
    """route + permute (one call) -> grouped SwiGLU FFN -> combine; y lands in buf['y'].
    With buf.gather the permute only sorts and the FFN reads x through perm;
    with buf.fused the combine also runs inside the FFN's down projection.
    With buf.aux_alpha the router's balancing loss lands in buf['aux_loss']."""
    t = buf.t
    B.moe_route_permute(shape, x, w_router, bias, t["logits"], t["topk_idx"], t["topk_w"],
                        t["offsets"], t["perm"], t["inv"], t["xp"], t["ws_route_permute"], stream)
    if buf.aux_alpha is not None:
        B.moe_aux_loss(shape, t["logits"], t["topk_idx"], buf.aux_alpha, t["aux_loss"], t["aux_w"],
                       t["ws_aux_loss"], stream)
    if buf.fused:  # combine included
        B.moe_grouped_ffn_fwd_fused(shape, x, t["perm"], t["inv"], t["topk_w"], t["offsets"],
                                    w_gate, w_up, w_down, t["h"], t["a"], t["yp"], t["y"],
                                    t["ws_ffn_fwd_fused"], stream)
        return
    if buf.gather:
        B.moe_grouped_ffn_fwd_gather(shape, x, t["perm"], t["offsets"], w_gate, w_up, w_down,
                                     t["h"], t["a"], t["yp"], t["ws_ffn_fwd"], stream)
    else:
        B.moe_grouped_ffn_fwd(shape, t["xp"], t["offsets"], w_gate, w_up, w_down, t["h"], t["a"],
                              t["yp"], t["ws_ffn_fwd"], stream)
    B.moe_combine(shape, t["yp"], t["inv"], t["topk_w"], t["y"], stream)


def small_path_fits(shape: B.MoEShape, training: bool) -> bool:
    """The size rule for the small-batch forward: inference only (it keeps no
    activations for a backward), no row capacity, and fewer than half as
    many routed (token, slot) pairs as local experts -- below that the sort,
    the tile tables and the grouped GEMMs' padded tiles cost more than the
    matrix-vector kernels (measured at the Qwen3-30B-A3B shape, E_loc = 128
    and k = 8: 41 vs 99 us at T = 1, 71 vs 103 at T = 4, 111 vs 107 at T = 8,
    so T <= 7 there)."""
    return (not training and shape.rows_cap == shape.T * shape.k
            and 2 * shape.T * shape.k < shape.E_loc
            and shape.T * shape.k <= B.SMALL_MAX_PAIRS
            and shape.d <= B.SMALL_MAX_WIDTH and shape.I <= B.SMALL_MAX_WIDTH)


def forward_small(shape: B.MoEShape, buf: LayerBuffers, x, w_router, bias, w_gate, w_up, w_down,
                  stream=None):
    """route -> small-batch FFN with the combine, in one call (no sort; for a
    few tokens); y lands in buf['y']."""
    t = buf.t
    if t.get("ws_small_routed_fwd") is None:
        t["ws_small_routed_fwd"] = buf._ws("small_routed_fwd")
    B.moe_small_fwd(shape, x, w_router, bias, t["logits"], t["topk_idx"], t["topk_w"], w_gate,
                    w_up, w_down, t["y"], t["ws_small_routed_fwd"], stream)


def forward_inference(shape: B.MoEShape, buf: LayerBuffers, x, w_router, bias, w_gate, w_up,
                      w_down, stream=None):
    """Inference forward by the size rule: the small-batch call for a few
    tokens, else the grouped path (the balancing loss is a training term and
    is not computed on the small path)."""
    if small_path_fits(shape, buf.training) and buf.aux_alpha is None:
        forward_small(shape, buf, x, w_router, bias, w_gate, w_up, w_down, stream)
    else:
        forward(shape, buf, x, w_router, bias, w_gate, w_up, w_down, stream)


def backward(shape: B.MoEShape, buf: LayerBuffers, dy, x, w_router, w_gate, w_up, w_down,
             stream=None):
    """combine_bwd -> grouped FFN bwd -> permute_bwd -> route_bwd (with the
    balancing loss's gradient when buf.aux_alpha is set)."""
    t = buf.t
    if buf.dy_form:  # dYp is the call's scratch, written only where a kernel reads it
        B.moe_combine_ffn_bwd_gather(shape, x, t["perm"], t["inv"], t["offsets"], t["topk_w"],
                                     w_gate, w_up, w_down, t["h"], t["a"], t["yp"], dy, t["dyp"],
                                     t["dtopk_w"], t["dxp"], t["dw_gate"], t["dw_up"],
                                     t["dw_down"], t["ws_ffn_bwd"], stream)
    elif buf.gather:
        B.moe_combine_bwd(shape, dy, t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"],
                          stream)
        B.moe_grouped_ffn_bwd_gather(shape, x, t["perm"], t["offsets"], w_gate, w_up, w_down,
                                     t["h"], t["a"], t["dyp"], t["dxp"], t["dw_gate"],
                                     t["dw_up"], t["dw_down"], t["ws_ffn_bwd"], stream)
    else:
        B.moe_combine_bwd(shape, dy, t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"],
                          stream)
        B.moe_grouped_ffn_bwd(shape, t["xp"], t["offsets"], w_gate, w_up, w_down, t["h"], t["a"],
                              t["dyp"], t["dxp"], t["dw_gate"], t["dw_up"], t["dw_down"],
                              t["ws_ffn_bwd"], stream)
    B.moe_permute_bwd(shape, t["dxp"], t["inv"], t["dx"], stream)
    if buf.aux_alpha is not None:
        B.moe_route_bwd_aux(shape, x, w_router, t["topk_idx"], t["topk_w"], t["dtopk_w"],
                            t["logits"], t["aux_w"], t["dlogits"], t["dw_router"], t["dbias"],
                            t["dx"], t["ws_route_bwd"], stream)
        return
    if shape.gate == B.GATES["balanced"]:
        # zero router gradients, already in the buffers (LayerBuffers)
        B.moe_route_bwd(shape, x, w_router, t["topk_idx"], t["topk_w"], t["dtopk_w"], None, None,
                        None, t["dx"], t["ws_route_bwd"], stream)
        return
    B.moe_route_bwd(shape, x, w_router, t["topk_idx"], t["topk_w"], t["dtopk_w"], t["dlogits"],
                    t["dw_router"], t["dbias"], t["dx"], t["ws_route_bwd"], stream)

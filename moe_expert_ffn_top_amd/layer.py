"""Buffers for one MoE layer call and the four-call sequence route -> group ->
expert_ffn -> combine.  PyTorch supplies device memory and streams only; every
step runs in libmoe's kernels."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B


@dataclass
class LayerBuffers:
    dims: B.Dims
    logits: torch.Tensor      # fp32 [T, E]
    ids: torch.Tensor         # int32 [T, k]
    w: torch.Tensor           # fp32 [T, k]
    sigma: torch.Tensor       # fp32 [T]
    offsets: torch.Tensor     # int32 [E+2]
    perm: torch.Tensor        # int32 [T*k]
    inv_perm: torch.Tensor    # int32 [T*k]
    group_slot: torch.Tensor  # int32 [E+1]
    status: torch.Tensor      # int32 [1]
    ws: torch.Tensor          # uint8 [moe_workspace_bytes]
    h: torch.Tensor           # bf16 [T*k+T, I]
    y_rows: torch.Tensor      # bf16 [T*k+T, H]
    y: torch.Tensor           # bf16 [T, H]
    mx_ws: Optional[torch.Tensor] = None  # uint8 [moe_mx_workspace_bytes]: MX blobs (moe_expert_ffn_mx)

    @staticmethod
    def allocate(dims: B.Dims, device="cuda", mx: bool = False) -> "LayerBuffers":
        T, H, I, E, k = dims.T, dims.H, dims.I, dims.E, dims.k
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        return LayerBuffers(
            dims=dims,
            logits=torch.empty((T, E), **f32), ids=torch.empty((T, k), **i32), w=torch.empty((T, k), **f32),
            sigma=torch.empty(T, **f32), offsets=torch.empty(E + 2, **i32), perm=torch.empty(T * k, **i32),
            inv_perm=torch.empty(T * k, **i32), group_slot=torch.empty(E + 1, **i32),
            status=torch.zeros(1, **i32),
            ws=torch.empty(B.moe_workspace_bytes(dims), dtype=torch.uint8, device=device),
            h=torch.empty((T * k + T, I), **bf), y_rows=torch.empty((T * k + T, H), **bf),
            y=torch.empty((T, H), **bf),
            mx_ws=torch.empty(B.moe_mx_workspace_bytes(dims), dtype=torch.uint8, device=device) if mx else None)


def run_layer(buf: LayerBuffers, layer: int, x: torch.Tensor, pool, pool_bytes: int, layout: B.BlobLayout,
              slot_table: torch.Tensor, n_slots: int, w_shared_gate: torch.Tensor,
              w_router: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None, stream=None,
              fused: bool = True) -> None:
    """Enqueue one layer on `stream` (default: torch's current stream).
    fused: route and group through moe_route_group (else moe_route then
    moe_group; the results are bit-identical)."""
    d = buf.dims
    lg_out = buf.logits if w_router is not None else None
    lg_in = None if w_router is not None else logits
    if fused:
        B.moe_route_group(d, layer, x, w_router, lg_in, w_shared_gate, lg_out, buf.ids, buf.w, buf.sigma, slot_table,
                          n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status, buf.ws,
                          stream=stream)
    else:
        B.moe_route(d, x, w_router, lg_in, w_shared_gate, lg_out, buf.ids, buf.w, buf.sigma, stream)
        B.moe_group(d, layer, buf.ids, slot_table, n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                    buf.status, buf.ws, stream=stream)
    if buf.mx_ws is not None:   # MX blobs: layout from moe_blob_layout_init_mx
        B.moe_expert_ffn_mx(d, x, pool, pool_bytes, layout, buf.offsets, buf.perm, buf.group_slot, buf.h, buf.y_rows,
                            buf.status, buf.ws, buf.mx_ws, stream=stream)
    else:
        B.moe_expert_ffn(d, x, pool, pool_bytes, layout, buf.offsets, buf.perm, buf.group_slot, buf.h, buf.y_rows,
                         buf.status, buf.ws, stream=stream)
    B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y, stream)

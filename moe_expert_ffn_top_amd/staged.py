"""Streamed layers through libmoe's two-slot staging ring.

Expert blobs of every layer live in page-locked host memory; each layer's
(E+1) blobs are copied into one of two device slots on a copy stream while
the previous layer computes on the compute stream ([Strata] "PCIe 搬运怎样与计算
重叠？"; [FreeToken] 3.1 full-layer double buffering).  The ring's events order
the streams; this module only sequences the calls."""
from __future__ import annotations

from typing import Callable, List, Optional

import torch

from . import binding as B
from .layer import LayerBuffers


class StagedLayers:
    def __init__(self, dims: B.Dims, layout: B.BlobLayout, host_pool: torch.Tensor, n_layers: int,
                 copy_stream: torch.cuda.Stream, compute_stream: torch.cuda.Stream):
        assert host_pool.is_pinned(), "host blobs must be page-locked"
        E1 = dims.E + 1
        self.dims, self.layout, self.L = dims, layout, n_layers
        self.layer_bytes = E1 * layout.slot_stride
        assert host_pool.numel() >= n_layers * self.layer_bytes
        self.host = host_pool
        self.copy_stream, self.compute_stream = copy_stream, compute_stream
        self.slots = [torch.empty(self.layer_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.ring = B.moe_ring_create(self.slots[0], self.slots[1], self.layer_bytes, copy_stream)
        # inside a slot, expert e of the layer sits at slot index e
        self.slot_table = torch.arange(E1, dtype=torch.int32, device="cuda").repeat(n_layers, 1).contiguous()
        self.buf = LayerBuffers.allocate(dims)

    def close(self) -> None:
        if self.ring:
            B.moe_ring_destroy(self.ring)
            self.ring = None

    def _stage(self, layer: int) -> int:
        src = self.host.data_ptr() + layer * self.layer_bytes
        return B.moe_stage_h2d(self.ring, src, self.layer_bytes)

    def run(self, x_of: Callable[[int], torch.Tensor], wsg_of: Callable[[int], torch.Tensor],
            logits_of: Callable[[int], Optional[torch.Tensor]], after_layer: Optional[Callable[[int], None]] = None,
            layer_events: Optional[List] = None) -> None:
        """Run all layers; after_layer(l) is called once layer l is enqueued
        (e.g. to snapshot outputs).  layer_events, if given, receives per layer
        (copy_start, copy_end, compute_start, compute_end) timing events."""
        d, buf = self.dims, self.buf
        cs = self.compute_stream
        pending = {}
        copy_ev = {}

        def stage(l):
            if layer_events is not None:
                a = torch.cuda.Event(enable_timing=True)
                a.record(self.copy_stream)
            pending[l] = self._stage(l)
            if layer_events is not None:
                b = torch.cuda.Event(enable_timing=True)
                b.record(self.copy_stream)
                copy_ev[l] = (a, b)

        stage(0)
        if self.L > 1:
            stage(1)
        for l in range(self.L):
            s = pending.pop(l)
            B.moe_ring_acquire(self.ring, s, cs)
            if layer_events is not None:
                c0 = torch.cuda.Event(enable_timing=True)
                c0.record(cs)
            pool = self.slots[s]
            x = x_of(l)
            lg = logits_of(l)
            B.moe_route(d, x, None, lg, wsg_of(l), None, buf.ids, buf.w, buf.sigma, cs)
            B.moe_group(d, l, buf.ids, self.slot_table, d.E + 1, buf.offsets, buf.perm, buf.inv_perm,
                        buf.group_slot, buf.status, buf.ws, stream=cs)
            B.moe_expert_ffn(d, x, pool, self.layer_bytes, self.layout, buf.offsets, buf.perm, buf.group_slot,
                             buf.h, buf.y_rows, buf.status, buf.ws, stream=cs)
            B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y, cs)
            if layer_events is not None:
                c1 = torch.cuda.Event(enable_timing=True)
                c1.record(cs)
            B.moe_ring_release(self.ring, s, cs)
            if layer_events is not None:
                layer_events.append((copy_ev[l][0], copy_ev[l][1], c0, c1))
            if after_layer is not None:
                after_layer(l)
            if l + 2 < self.L:
                stage(l + 2)

    def run_serial(self, x_of: Callable[[int], torch.Tensor], wsg_of: Callable[[int], torch.Tensor],
                   logits_of: Callable[[int], Optional[torch.Tensor]]) -> None:
        """The reference without the second buffer: one slot, and on the
        compute stream each layer's copy, then its compute, so no copy overlaps
        any compute ([FreeToken] 5.3 measures what the second buffer buys).
        The ring is not used."""
        d, buf = self.dims, self.buf
        cs = self.compute_stream
        pool = self.slots[0]
        for l in range(self.L):
            src = self.host[l * self.layer_bytes:(l + 1) * self.layer_bytes]
            with torch.cuda.stream(cs):
                pool.copy_(src, non_blocking=True)
            x = x_of(l)
            B.moe_route(d, x, None, logits_of(l), wsg_of(l), None, buf.ids, buf.w, buf.sigma, cs)
            B.moe_group(d, l, buf.ids, self.slot_table, d.E + 1, buf.offsets, buf.perm, buf.inv_perm,
                        buf.group_slot, buf.status, buf.ws, stream=cs)
            B.moe_expert_ffn(d, x, pool, self.layer_bytes, self.layout, buf.offsets, buf.perm, buf.group_slot,
                             buf.h, buf.y_rows, buf.status, buf.ws, stream=cs)
            B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y, cs)

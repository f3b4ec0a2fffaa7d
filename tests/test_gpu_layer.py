"""GPU tests of moe_route_group_ffn_combine: route, group, both expert FFN
stages and the combine in one call; for decode windows with drawn logits the
whole layer is one launch ([FreeToken] 3.5: one step's control flow on the
device).  Every workgroup routes the window for itself; one stores the
routing outputs, zeroes the launch's counters and raises a ready flag; the
down items wait inside the launch for their tiles' h rows, and the wavefront
that completes a block of output columns combines it ([Strata]
"路由以后，专家怎样分工？").

- Against moe_route_group, moe_expert_ffn and moe_combine launched apart:
  ids, weights, sigma, offsets, perm, inv_perm, group_slot, status, the live
  rows of h and Y, and y, all bit for bit, on two calls in a row; the
  decode48 shape also against the oracle.
- Shapes: the three (H, I) pairs with a one-launch instantiation (2048 x 512
  with the 48-layer decode window, 4096 x 2048 with the 43-layer one, 512 x
  256 with T k from 3 to 256 and E up to 1000), and shapes that run the
  separate launches (k > 16; an (H, I) without an instantiation; the router
  matrix).
- A workspace fresh from the allocator (every byte 0xFF, then random bytes):
  the launch zeroes its own counters before counting, so the results are the
  same.
- A routed and the shared expert not resident: status bits and zero rows.
- The layer captured in a HIP graph, replayed with eager work between.
- A wait forced to time out from the host (tile targets never reached, a
  small poll limit): MOE_DEV_SYNC_TIMEOUT is set, every wavefront ends, and
  the next call is correct again."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say
from oracle import moe_oracle as O
from synth import Config
from test_gpu_fused import FCase
from test_gpu_route_ffn import assert_same, scramble, separate, snapshot

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


CASES = {
    "decode48_shape": Config(101, "l1", T=4, H=2048, I=512, E=512, k=10, L=1, router="zipf", zipf_s=1.0),
    "decode43_shape": Config(102, "l2", T=16, H=4096, I=2048, E=256, k=6, L=1, router="zipf", zipf_s=1.2),
    "h512_i256": Config(103, "l3", T=8, H=512, I=256, E=32, k=4, L=1, router="zipf", zipf_s=0.8),
    "one_token": Config(104, "l4", T=1, H=512, I=256, E=96, k=3, L=1, router="zipf", zipf_s=1.0),
    "f65": Config(105, "l5", T=13, H=512, I=256, E=40, k=5, L=1, router="zipf", zipf_s=0.7),
    "f256": Config(106, "l6", T=16, H=512, I=256, E=64, k=16, L=1, router="zipf", zipf_s=1.0),
    "e1000": Config(107, "l7", T=3, H=512, I=256, E=1000, k=7, L=1, router="zipf", zipf_s=1.1),
    "one_expert": Config(108, "l8", T=5, H=512, I=256, E=1, k=1, L=1, router="zipf", zipf_s=1.0),
    # separate launches: k > 16, and (H, I) without a one-launch instantiation
    "k20_separate": Config(109, "l9", T=10, H=512, I=256, E=1000, k=20, L=1, router="zipf", zipf_s=1.1),
    "h256_separate": Config(110, "l10", T=16, H=256, I=128, E=1024, k=16, L=1, router="zipf", zipf_s=0.9),
}


def layer_call(B, c):
    b = c.buf
    lg_out = b.logits if c.wr_t is not None else None
    B.moe_route_group_ffn_combine(c.d, 0, c.x, c.wr_t, c.lg_t, c.wsg_t, lg_out, b.ids, b.w, b.sigma, c.st,
                                  c.cfg.E1, b.offsets, b.perm, b.inv_perm, b.group_slot, c.pool, c.pool_bytes, c.lay,
                                  b.h, b.y_rows, b.y, b.status, b.ws)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_matches_separate_launches(B, hostgen, name):
    cfg = CASES[name]
    say("[gpu] one-launch layer %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    assert int(want["status"].item()) == 0
    for rep in range(2):
        scramble(c)
        layer_call(B, c)
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "call %d" % rep)
    if name != "decode48_shape":
        return
    ora = O.moe_layer(c.x_bits, lambda e: c.blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, c.wsg, logits=c.lg)
    stats = compare_layer(c.buf, ora, cfg.T, cfg.k, cfg.E, drawn_logits=True)
    say("[gpu]   %s against the oracle: %s" % (name, stats))


def test_layer_router_matrix_runs_separately(B, hostgen):
    cfg = Config(111, "l11", T=8, H=512, I=256, E=32, k=4, L=1, router="matrix")
    say("[gpu] one-launch layer with the router matrix (separate kernels)")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    scramble(c)
    layer_call(B, c)
    torch.cuda.synchronize()
    assert_same(snapshot(c), want, "router matrix")


@pytest.mark.parametrize("name", ["decode48_shape", "h512_i256"])
def test_layer_fresh_workspace(B, hostgen, name):
    cfg = CASES[name]
    say("[gpu] one-launch layer %s on a workspace of garbage bytes" % name)
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for fill in ("ff", "random"):
        ws = c.buf.ws
        if fill == "ff":
            ws.view(torch.uint8).fill_(0xFF)
        else:
            ws.view(torch.uint8).copy_(torch.randint(0, 256, (ws.numel() * ws.element_size(),), dtype=torch.uint8,
                                                     device="cuda", generator=gen))
        scramble(c)
        layer_call(B, c)
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "workspace %s" % fill)


def test_layer_non_resident(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] one-launch layer: a routed and the shared expert not resident")
    probe = FCase(B, cfg, hostgen)
    probe.route_group(B)
    torch.cuda.synchronize()
    off = probe.buf.offsets.cpu().numpy()
    e = int(np.argmax(np.diff(off[:cfg.E + 1])))   # a routed expert with rows
    c = FCase(B, cfg, hostgen, slot_override={e: -1, cfg.E: -1})
    want = separate(B, c)
    assert int(want["status"].item()) & B.MOE_DEV_NOT_RESIDENT
    scramble(c)
    layer_call(B, c)
    torch.cuda.synchronize()
    got = snapshot(c)
    assert_same(got, want, "non-resident")
    assert not int(got["status"].item()) & B.MOE_DEV_SYNC_TIMEOUT
    assert torch.count_nonzero(c.buf.h[off[e]:off[e + 1]].float()) == 0
    assert torch.count_nonzero(c.buf.y_rows[cfg.T * cfg.k:cfg.T * cfg.k + cfg.T].float()) == 0


def test_layer_graph_replays(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] one-launch layer in a HIP graph")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer_call(B, c)
    for _ in range(3):
        scramble(c)
        c.route_group(B)   # eager work between the replays
        c.ffn(B, stages=1)
        torch.cuda.synchronize()
        scramble(c)
        g.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "graph replay")


def test_layer_wait_timeout_is_flagged_and_recovers(B, hostgen):
    cfg = CASES["h512_i256"]
    say("[gpu] one-launch layer: a wait forced to time out")
    lib = ctypes.CDLL(B.LIB_PATH)
    lib.moe_debug_set_fused_wait.argtypes = [ctypes.c_int, ctypes.c_int]
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    try:
        lib.moe_debug_set_fused_wait(8, 1)   # the tile targets are never reached; 8 polls each
        c.buf.status.zero_()
        layer_call(B, c)
        torch.cuda.synchronize()
        assert int(c.buf.status.item()) & B.MOE_DEV_SYNC_TIMEOUT
    finally:
        lib.moe_debug_set_fused_wait(-1, 0)
    scramble(c)
    layer_call(B, c)
    torch.cuda.synchronize()
    assert_same(snapshot(c), want, "after the time-out")

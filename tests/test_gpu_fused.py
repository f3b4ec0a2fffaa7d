"""GPU tests of the one-launch decode FFN (moe_expert_ffn_combine: both stages
and the combine in one persistent launch whose down items wait inside the
launch for the gate/up items that write their h rows; [FreeToken] 3.5, one
step's control flow on the device).

- moe_expert_ffn_combine against the two stages launched apart
  (moe_expert_ffn_stages 1 then 2) and moe_combine: h, Y and y bit for bit,
  and y against the oracle;
- a second call with the same grouping (the launch resets its counters);
- many more items than workgroups (each walks several, and several down
  items wait);
- a non-resident group (zero rows, the status bit, the others unchanged);
- the step captured in a HIP graph, replayed with eager work between;
- a wait forced to time out from the host (a target the counters never
  reach, a small poll limit): MOE_DEV_SYNC_TIMEOUT is set, every wavefront
  ends, and the next call is correct again."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say
from oracle import moe_oracle as O
from synth import Config, HostGen, zipf_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


# the three (H, I) shapes with a one-launch instantiation, plus a window whose
# tiles outnumber the grid many times
CASES = {
    "h512_i256": Config(71, "f1", T=8, H=512, I=256, E=32, k=4, L=1, router="matrix"),
    "decode48_shape": Config(72, "f2", T=4, H=2048, I=512, E=512, k=10, L=1, router="zipf", zipf_s=1.0),
    "decode43_shape": Config(73, "f3", T=16, H=4096, I=2048, E=48, k=6, L=1, router="zipf", zipf_s=1.2),
    "many_tiles": Config(74, "f4", T=64, H=2048, I=512, E=256, k=8, L=1, router="zipf", zipf_s=0.6),
}


class FCase:
    """One layer: the pool generated on the device (the device generator equals
    the host one byte for byte, tests/test_gpu_full.py); the oracle's blobs
    generated on the host as it asks for them."""

    def __init__(self, B, cfg, gen, slot_override=None):
        from moe_expert_ffn_top_amd.layer import LayerBuffers
        from synth import DevGen
        self.cfg = cfg
        self.d = B.Dims(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, 1)
        self.lay = B.moe_blob_layout_init(cfg.H, cfg.I)
        olay = O.blob_layout(cfg.H, cfg.I)
        E1 = cfg.E1
        self.blobs = _Lazy(lambda e: gen.expert_blob(cfg, 0, e, olay))
        self.pool_bytes = E1 * self.lay.slot_stride
        self.pool = torch.zeros(self.pool_bytes, dtype=torch.uint8, device="cuda")
        ident = torch.arange(E1, dtype=torch.int32, device="cuda").view(1, E1).contiguous()
        DevGen().pool(cfg, 0, 1, ident.data_ptr(), E1, self.lay, self.pool.data_ptr())
        torch.cuda.synchronize()
        st = np.arange(E1, dtype=np.int32)[None, :].copy()
        for e, s in (slot_override or {}).items():
            st[0, e] = s
        self.st = torch.from_numpy(st).cuda()
        self.x_bits = gen.x(cfg, 0, 0)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        self.wsg = gen.w_shared_gate(cfg, 0)
        self.wsg_t = torch.from_numpy(self.wsg).cuda()
        if cfg.router == "matrix":
            self.wr = gen.w_router(cfg, 0)
            self.wr_t = torch.from_numpy(self.wr).cuda()
            self.lg, self.lg_t = None, None
        else:
            self.wr, self.wr_t = None, None
            self.lg = zipf_logits(cfg, 0, 0)
            self.lg_t = torch.from_numpy(self.lg).cuda()
        self.buf = LayerBuffers.allocate(self.d)

    def route_group(self, B):
        b = self.buf
        B.moe_route_group(self.d, 0, self.x, self.wr_t, self.lg_t, self.wsg_t,
                          b.logits if self.wr_t is not None else None, b.ids, b.w, b.sigma, self.st, self.cfg.E1,
                          b.offsets, b.perm, b.inv_perm, b.group_slot, b.status, b.ws)

    def ffn(self, B, stages=None, combine=False):
        b = self.buf
        if combine:
            B.moe_expert_ffn_combine(self.d, self.x, self.pool, self.pool_bytes, self.lay, b.offsets, b.perm,
                                     b.group_slot, b.inv_perm, b.w, b.sigma, b.h, b.y_rows, b.y, b.status, b.ws)
        elif stages is None:
            B.moe_expert_ffn(self.d, self.x, self.pool, self.pool_bytes, self.lay, b.offsets, b.perm, b.group_slot,
                             b.h, b.y_rows, b.status, b.ws)
        else:
            B.moe_expert_ffn_stages(self.d, self.x, self.pool, self.pool_bytes, self.lay, b.offsets, b.perm,
                                    b.group_slot, b.h, b.y_rows, b.status, b.ws, stages)

    def combine(self, B):
        b = self.buf
        B.moe_combine(self.d, b.y_rows, b.inv_perm, b.w, b.sigma, b.y)

    def outputs(self):
        """h and Y of the live rows, and y, as int16 bit patterns."""
        b, c = self.buf, self.cfg
        off_e = int(b.offsets[c.E].item())
        live = torch.cat([torch.arange(off_e), torch.arange(c.T * c.k, c.T * c.k + c.T)]).cuda()
        return (b.h.view(torch.int16)[live].clone(), b.y_rows.view(torch.int16)[live].clone(),
                b.y.view(torch.int16).clone())

    def scramble(self):
        for t in (self.buf.h, self.buf.y_rows, self.buf.y):
            t.fill_(3.0)


class _Lazy(dict):
    def __init__(self, make):
        super().__init__()
        self.make = make

    def __missing__(self, e):
        v = self[e] = self.make(e)
        return v


def _same(a, b, what):
    for u, v, n in zip(a, b, ("h", "Y rows", "y")):
        assert torch.equal(u, v), "%s: %s differs" % (what, n)


@pytest.mark.parametrize("name", list(CASES))
def test_one_launch_matches_split_stages_and_combine(B, hostgen, name):
    cfg = CASES[name]
    say("[gpu] one-launch FFN %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = FCase(B, cfg, hostgen)
    c.route_group(B)
    c.scramble()
    c.ffn(B, stages=1)
    c.ffn(B, stages=2)
    c.combine(B)
    torch.cuda.synchronize()
    assert int(c.buf.status.item()) == 0
    want = c.outputs()
    for rep in range(2):   # the second call reuses the grouping: the launch reset its counters
        c.scramble()
        c.ffn(B)
        c.combine(B)
        torch.cuda.synchronize()
        _same(c.outputs(), want, "moe_expert_ffn + moe_combine, call %d" % rep)
        c.scramble()
        c.ffn(B, combine=True)
        torch.cuda.synchronize()
        _same(c.outputs(), want, "moe_expert_ffn_combine, call %d" % rep)
    assert int(c.buf.status.item()) == 0
    if cfg.H * cfg.I > 2048 * 512:
        return   # the split path is held to the oracle at this shape in tests/test_gpu_full.py
    # and the layer against the oracle
    ora = O.moe_layer(c.x_bits, lambda e: c.blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, c.wsg, w_router=c.wr,
                      logits=c.lg)
    stats = compare_layer(c.buf, ora, cfg.T, cfg.k, cfg.E, drawn_logits=c.lg is not None,
                          x64=O.bf16_bits_to_f64(c.x_bits), w_router=c.wr)
    say("[gpu]   %s ok: %s" % (name, stats))


def test_one_launch_non_resident_group(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] one-launch FFN with a non-resident group")
    full = FCase(B, cfg, hostgen)
    full.route_group(B)
    full.ffn(B, combine=True)
    torch.cuda.synchronize()
    off = full.buf.offsets.cpu().numpy()
    e = int(np.argmax(np.diff(off[:cfg.E + 1])))   # a routed expert with rows
    c = FCase(B, cfg, hostgen, slot_override={e: -1})
    c.route_group(B)
    c.ffn(B, combine=True)
    torch.cuda.synchronize()
    assert int(c.buf.status.item()) & B.MOE_DEV_NOT_RESIDENT
    assert not int(c.buf.status.item()) & B.MOE_DEV_SYNC_TIMEOUT
    assert torch.count_nonzero(c.buf.y_rows[off[e]:off[e + 1]].float()) == 0
    assert torch.count_nonzero(c.buf.h[off[e]:off[e + 1]].float()) == 0
    keep = torch.ones(cfg.T * cfg.k + cfg.T, dtype=torch.bool, device="cuda")
    keep[off[e]:off[e + 1]] = False
    assert torch.equal(c.buf.y_rows[keep].view(torch.int16), full.buf.y_rows[keep].view(torch.int16))
    # the combine of the fused launch equals moe_combine over the same rows
    y1 = c.buf.y.view(torch.int16).clone()
    c.combine(B)
    torch.cuda.synchronize()
    assert torch.equal(c.buf.y.view(torch.int16), y1)


def test_one_launch_graph_replays(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] one-launch FFN + combine in a HIP graph")
    c = FCase(B, cfg, hostgen)
    c.route_group(B)
    c.ffn(B, combine=True)
    torch.cuda.synchronize()
    want = c.outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.route_group(B)
        c.ffn(B, combine=True)
    for _ in range(3):
        c.scramble()
        c.route_group(B)   # eager work between the replays
        c.ffn(B, stages=1)
        torch.cuda.synchronize()
        c.scramble()
        g.replay()
        torch.cuda.synchronize()
        _same(c.outputs(), want, "graph replay")
    assert int(c.buf.status.item()) == 0


def test_one_launch_wait_timeout_is_flagged_and_recovers(B, hostgen):
    cfg = CASES["h512_i256"]
    say("[gpu] one-launch FFN: a wait forced to time out")
    lib = ctypes.CDLL(B.LIB_PATH)
    lib.moe_debug_set_fused_wait.argtypes = [ctypes.c_int, ctypes.c_int]
    c = FCase(B, cfg, hostgen)
    c.route_group(B)
    c.ffn(B, stages=1)
    c.ffn(B, stages=2)
    torch.cuda.synchronize()
    want = c.outputs()[:2]
    try:
        lib.moe_debug_set_fused_wait(8, 1)   # the tile targets are never reached; 8 polls each
        c.buf.status.zero_()
        c.ffn(B, combine=True)
        torch.cuda.synchronize()
        assert int(c.buf.status.item()) & B.MOE_DEV_SYNC_TIMEOUT
    finally:
        lib.moe_debug_set_fused_wait(-1, 0)
    c.buf.status.zero_()
    c.scramble()
    c.ffn(B, combine=True)
    torch.cuda.synchronize()
    assert int(c.buf.status.item()) == 0
    got = c.outputs()[:2]
    assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])

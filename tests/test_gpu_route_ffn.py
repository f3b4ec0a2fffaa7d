"""GPU tests of moe_route_group_ffn: route + group + expert FFN in one call; for
decode windows with drawn logits the routing runs inside the gate/up launch
([FreeToken] 3.5: one step's control flow on the device), every workgroup
grouping the window for itself and one more storing the routing outputs.

- Against moe_route_group then moe_expert_ffn (and moe_combine after both):
  ids, weights, sigma, offsets, perm, inv_perm, group_slot, status, the live
  rows of h and Y, and y, all bit for bit; the decode48 shape also against the
  oracle.
- Shapes: the 48-layer decode window (T = 4, k = 10, E = 512); T k = 64 (one
  sorting wavefront's limit); the 43-layer decode window's routing (T = 16,
  k = 6, E = 256: two sorting wavefronts); T k = 65 (a second wavefront with
  one row); T k = 256 (four wavefronts, groups of up to 16 rows); T k = 200
  with E = 1000; T k = 256 with E = 1024 (the largest window and pool); one
  expert (E = 1, k = 1: one group of every token); one token; E = 1000 (16
  logits per lane, not a multiple of 64); H = 512, I = 256.
- A routed expert and the shared expert not resident: the status bits and zero
  rows, as on the separate path.
- stages = 1, then the down stage on its own.
- The step captured in a HIP graph, replayed with eager work between.
- The router matrix (w_router): the separate kernels, the same results.
- Tied logits (a half-unit grid; one token with every logit equal, which
  leaves more than 64 candidates at the threshold; -0 beside +0): the same
  winners and slot order as the separate launches, and as the oracle's top-k."""
import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say
from oracle import moe_oracle as O
from synth import Config
from test_gpu_fused import FCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


CASES = {
    "decode48_shape": Config(81, "r1", T=4, H=2048, I=512, E=512, k=10, L=1, router="zipf", zipf_s=1.0),
    "h512_i256": Config(82, "r2", T=8, H=512, I=256, E=32, k=4, L=1, router="zipf", zipf_s=0.8),
    "f64": Config(83, "r3", T=16, H=512, I=256, E=64, k=4, L=1, router="zipf", zipf_s=1.2),
    "one_token": Config(84, "r4", T=1, H=512, I=256, E=96, k=3, L=1, router="zipf", zipf_s=1.0),
    "e1000": Config(85, "r5", T=3, H=512, I=256, E=1000, k=7, L=1, router="zipf", zipf_s=1.1),
    "f96_decode43_routing": Config(87, "r7", T=16, H=512, I=256, E=256, k=6, L=1, router="zipf", zipf_s=1.2),
    "f65": Config(88, "r8", T=13, H=512, I=256, E=40, k=5, L=1, router="zipf", zipf_s=0.7),
    "f256": Config(89, "r9", T=16, H=512, I=256, E=64, k=16, L=1, router="zipf", zipf_s=1.0),
    "f200_e1000": Config(90, "r10", T=10, H=512, I=256, E=1000, k=20, L=1, router="zipf", zipf_s=1.1),
    "one_expert": Config(92, "r12", T=5, H=512, I=256, E=1, k=1, L=1, router="zipf", zipf_s=1.0),
    "e1024_f256": Config(93, "r13", T=16, H=256, I=128, E=1024, k=16, L=1, router="zipf", zipf_s=0.9),
}


def route_group_ffn(B, c, stages=3):
    b = c.buf
    lg_out = b.logits if c.wr_t is not None else None
    B.moe_route_group_ffn(c.d, 0, c.x, c.wr_t, c.lg_t, c.wsg_t, lg_out, b.ids, b.w, b.sigma, c.st, c.cfg.E1,
                          b.offsets, b.perm, b.inv_perm, b.group_slot, c.pool, c.pool_bytes, c.lay, b.h, b.y_rows,
                          b.status, b.ws, stages)


def snapshot(c):
    """Every output, as int32 / int16 bit patterns; h and Y on the rows a call
    writes (routed rows of groups, then the shared group's)."""
    b, cfg = c.buf, c.cfg
    off = b.offsets.clone()
    live = torch.cat([torch.arange(int(off[cfg.E].item())), torch.arange(cfg.T * cfg.k, cfg.T * cfg.k + cfg.T)])
    live = live.cuda()
    return dict(ids=b.ids.clone(), w=b.w.view(torch.int32).clone(), sigma=b.sigma.view(torch.int32).clone(),
                offsets=off, perm=b.perm.clone(), inv_perm=b.inv_perm.clone(), group_slot=b.group_slot.clone(),
                status=b.status.clone(), h=b.h.view(torch.int16)[live].clone(),
                y_rows=b.y_rows.view(torch.int16)[live].clone(), y=b.y.view(torch.int16).clone())


def scramble(c):
    b = c.buf
    for t in (b.ids, b.offsets, b.perm, b.inv_perm, b.group_slot):
        t.fill_(-5)
    for t in (b.w, b.sigma):
        t.fill_(7.0)
    for t in (b.h, b.y_rows, b.y):
        t.fill_(3.0)
    b.status.zero_()


def assert_same(got, want, what):
    for k in want:
        assert torch.equal(got[k], want[k]), "%s: %s differs" % (what, k)


def separate(B, c):
    c.route_group(B)
    c.ffn(B)
    c.combine(B)
    torch.cuda.synchronize()
    return snapshot(c)


@pytest.mark.parametrize("name", list(CASES))
def test_route_group_ffn_matches_separate_launches(B, hostgen, name):
    cfg = CASES[name]
    say("[gpu] route + group + FFN %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    assert int(want["status"].item()) == 0
    for rep in range(2):
        scramble(c)
        route_group_ffn(B, c)
        c.combine(B)
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "call %d" % rep)
    if name != "decode48_shape":
        return
    ora = O.moe_layer(c.x_bits, lambda e: c.blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, c.wsg, logits=c.lg)
    stats = compare_layer(c.buf, ora, cfg.T, cfg.k, cfg.E, drawn_logits=True)
    say("[gpu]   %s against the oracle: %s" % (name, stats))


def test_route_group_ffn_non_resident(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] route + group + FFN: a routed and the shared expert not resident")
    probe = FCase(B, cfg, hostgen)
    probe.route_group(B)
    torch.cuda.synchronize()
    off = probe.buf.offsets.cpu().numpy()
    e = int(np.argmax(np.diff(off[:cfg.E + 1])))   # a routed expert with rows
    c = FCase(B, cfg, hostgen, slot_override={e: -1, cfg.E: -1})
    want = separate(B, c)
    assert int(want["status"].item()) & B.MOE_DEV_NOT_RESIDENT
    scramble(c)
    route_group_ffn(B, c)
    c.combine(B)
    torch.cuda.synchronize()
    got = snapshot(c)
    assert_same(got, want, "non-resident")
    assert torch.count_nonzero(c.buf.h[off[e]:off[e + 1]].float()) == 0
    assert torch.count_nonzero(c.buf.y_rows[cfg.T * cfg.k:cfg.T * cfg.k + cfg.T].float()) == 0


def test_route_group_ffn_gate_up_then_down(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] route + group + FFN, stages = 1, then the down stage")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    scramble(c)
    route_group_ffn(B, c, stages=1)
    c.ffn(B, stages=2)
    c.combine(B)
    torch.cuda.synchronize()
    assert_same(snapshot(c), want, "stages 1 + 2")


def test_route_group_ffn_graph_replays(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] route + group + FFN in a HIP graph")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        route_group_ffn(B, c)
        c.combine(B)
    for _ in range(3):
        scramble(c)
        c.route_group(B)   # eager work between the replays
        c.ffn(B, stages=1)
        torch.cuda.synchronize()
        scramble(c)
        g.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "graph replay")


def test_route_group_ffn_router_matrix_runs_separately(B, hostgen):
    cfg = Config(86, "r6", T=8, H=512, I=256, E=32, k=4, L=1, router="matrix")
    say("[gpu] route + group + FFN with the router matrix (separate kernels)")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    scramble(c)
    route_group_ffn(B, c)
    c.combine(B)
    torch.cuda.synchronize()
    assert_same(snapshot(c), want, "router matrix")


@pytest.mark.parametrize("T,E,k", [(4, 512, 10), (16, 256, 6), (13, 40, 5), (16, 64, 16)])
def test_route_group_ffn_tied_logits(B, hostgen, T, E, k):
    cfg = Config(91, "r11", T=T, H=512, I=256, E=E, k=k, L=1, router="zipf", zipf_s=1.0)
    say("[gpu] route + group + FFN on tied logits (T=%d E=%d k=%d)" % (T, E, k))
    c = FCase(B, cfg, hostgen)
    rng = np.random.default_rng(T * 131 + E + k)
    lg = (np.round(rng.normal(size=(T, E)) * 2) / 2).astype(np.float32)
    lg[0, :] = 0.25
    if T > 1:
        lg[1, 0::2] = -0.0
        lg[1, 1::2] = 0.0
    c.lg = lg
    c.lg_t = torch.from_numpy(lg).cuda()
    want = separate(B, c)
    assert np.array_equal(want["ids"].cpu().numpy(), O.topk(lg, k))
    for rep in range(2):
        scramble(c)
        route_group_ffn(B, c)
        c.combine(B)
        torch.cuda.synchronize()
        assert_same(snapshot(c), want, "tied logits, call %d" % rep)

"""GPU tests of moe_expert_ffn_down_combine: the down stage and the combine in
one call ([Strata] "路由以后，专家怎样分工？": a token's expert outputs are
weighted and summed once all of them have arrived).  On decode windows with
I = 512 it is one launch in which two workgroups share each block of 16 output
columns and the second to finish combines it; elsewhere the two launches.

- Against moe_expert_ffn (both stages) then moe_combine: the live rows of Y and
  y, bit for bit, after the gate/up stage of moe_route_group_ffn (routing in
  the launch) and after moe_route_group + moe_expert_ffn_stages(1).
- Shapes: the 48-layer decode window (T = 4, k = 10, E = 512, H = 2048,
  I = 512); T = 16, k = 16 (256 entries, tiles of up to 16 rows); T = 13,
  k = 5 (odd tile counts); one token; one expert; a shape the one launch does
  not take (I = 256: the two launches).
- Two calls in a row on the same work list (the block counters are zeroed
  again after each use), and the decode48 shape against the oracle.
- A routed expert and the shared expert not resident: zero rows, as on the
  separate path.
- The layer captured in a HIP graph and replayed with eager work between."""
import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say
from oracle import moe_oracle as O
from synth import Config
from test_gpu_fused import FCase
from test_gpu_route_ffn import route_group_ffn, scramble, separate, snapshot

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


CASES = {
    "decode48_shape": Config(81, "r1", T=4, H=2048, I=512, E=512, k=10, L=1, router="zipf", zipf_s=1.0),
    "t16_k16": Config(301, "dc2", T=16, H=512, I=512, E=64, k=16, L=1, router="zipf", zipf_s=1.0),
    "t13_k5": Config(302, "dc3", T=13, H=1024, I=512, E=40, k=5, L=1, router="zipf", zipf_s=0.7),
    "one_token": Config(303, "dc4", T=1, H=512, I=512, E=96, k=3, L=1, router="zipf", zipf_s=1.0),
    "one_expert": Config(304, "dc5", T=5, H=512, I=512, E=1, k=1, L=1, router="zipf", zipf_s=1.0),
    "i256_two_launches": Config(82, "r2", T=8, H=512, I=256, E=32, k=4, L=1, router="zipf", zipf_s=0.8),
}


def down_combine(B, c):
    b = c.buf
    B.moe_expert_ffn_down_combine(c.d, c.x, c.pool, c.pool_bytes, c.lay, b.offsets, b.perm, b.group_slot,
                                  b.inv_perm, b.w, b.sigma, b.h, b.y_rows, b.y, b.status, b.ws)


@pytest.mark.parametrize("name", list(CASES))
def test_down_combine_matches_separate_launches(B, hostgen, name):
    cfg = CASES[name]
    say("[gpu] down + combine %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    assert int(want["status"].item()) == 0
    for rep in range(2):
        # routing inside the gate/up launch, then the new call (twice on the
        # same work list: the counters are zeroed again after each use)
        scramble(c)
        route_group_ffn(B, c, stages=1)
        down_combine(B, c)
        if rep == 1:
            c.buf.y.fill_(3.0)
            down_combine(B, c)
        torch.cuda.synchronize()
        assert_same = snapshot(c)
        for k in ("y_rows", "y", "h", "status"):
            assert torch.equal(assert_same[k], want[k]), "call %d: %s differs" % (rep, k)
    # the separate routing kernels, then gate/up on its own, then the new call
    scramble(c)
    c.route_group(B)
    c.ffn(B, stages=1)
    down_combine(B, c)
    torch.cuda.synchronize()
    got = snapshot(c)
    for k in ("y_rows", "y"):
        assert torch.equal(got[k], want[k]), "after moe_route_group: %s differs" % k
    if name != "decode48_shape":
        return
    ora = O.moe_layer(c.x_bits, lambda e: c.blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, c.wsg, logits=c.lg)
    stats = compare_layer(c.buf, ora, cfg.T, cfg.k, cfg.E, drawn_logits=True)
    say("[gpu]   %s against the oracle: %s" % (name, stats))


def test_down_combine_non_resident(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] down + combine: a routed and the shared expert not resident")
    probe = FCase(B, cfg, hostgen)
    probe.route_group(B)
    torch.cuda.synchronize()
    off = probe.buf.offsets.cpu().numpy()
    e = int(np.argmax(np.diff(off[:cfg.E + 1])))
    c = FCase(B, cfg, hostgen, slot_override={e: -1, cfg.E: -1})
    want = separate(B, c)
    scramble(c)
    route_group_ffn(B, c, stages=1)
    down_combine(B, c)
    torch.cuda.synchronize()
    got = snapshot(c)
    for k in ("y_rows", "y", "status"):
        assert torch.equal(got[k], want[k]), "non-resident: %s differs" % k
    assert torch.count_nonzero(c.buf.y_rows[off[e]:off[e + 1]].float()) == 0
    assert torch.count_nonzero(c.buf.y_rows[cfg.T * cfg.k:cfg.T * cfg.k + cfg.T].float()) == 0


def test_down_combine_graph_replays(B, hostgen):
    cfg = CASES["decode48_shape"]
    say("[gpu] down + combine captured in a graph, replayed with eager work between")
    c = FCase(B, cfg, hostgen)
    want = separate(B, c)
    scramble(c)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        route_group_ffn(B, c, stages=1)
        down_combine(B, c)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        route_group_ffn(B, c, stages=1)
        down_combine(B, c)
    for rep in range(3):
        scramble(c)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(c)
        for k in ("y_rows", "y", "h"):
            assert torch.equal(got[k], want[k]), "replay %d: %s differs" % (rep, k)
        # eager work between replays
        c.route_group(B)
        c.ffn(B)
        torch.cuda.synchronize()

"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same kernels and grids; the benchmark replays the same calls
from HIP graphs, checked here to be bit-identical to eager launches).

Routing and grouping are compared for every token of the sampled layers;
the expert rows and outputs for sampled tokens, which the oracle computes one
by one (a token's output depends only on its own row, its routing and the
expert bytes).  The oracle reads expert bytes from the host generator; a test
checks that the device generator that filled the GPU pool wrote the same
bytes."""
import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say
from oracle import moe_oracle as O
from synth import CONFIGS, DevGen, HostGen, zipf_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


def _snapshot(buf):
    return type("Snap", (), {k: getattr(buf, k).clone() for k in
                             ("ids", "w", "sigma", "offsets", "perm", "inv_perm", "h", "y_rows", "y", "logits",
                              "status")})


def _oracle_layer(cfg, gen, layer, step, tokens, wl_logits=None):
    olay = O.blob_layout(cfg.H, cfg.I)
    x = gen.x(cfg, layer, step)
    wsg = gen.w_shared_gate(cfg, layer)
    if cfg.router == "matrix":
        wr = gen.w_router(cfg, layer)
        lg = O.router_logits(O.bf16_bits_to_f64(x), wr)
        kw = dict(w_router=wr)
    else:
        wr = None
        lg = zipf_logits(cfg, layer, step)
        kw = dict(logits=lg)
    need = set(O.topk(lg[list(tokens)], cfg.k).reshape(-1).tolist()) | {cfg.E}
    blobs = {e: gen.expert_blob(cfg, layer, e, olay) for e in need}
    return O.moe_layer(x, lambda e: blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, wsg, tokens=tokens, **kw), x, wr


def _check_device_generator(wl, cfg, gen, layer, experts, step=0):
    olay = O.blob_layout(cfg.H, cfg.I)
    stride = wl.layout.slot_stride
    for e in experts:
        slot = layer * cfg.E1 + e
        dev = wl.pool[slot * stride: slot * stride + olay.blob_bytes].cpu().numpy()
        host = gen.expert_blob(cfg, layer, e, olay)[:olay.blob_bytes]
        assert np.array_equal(dev, host), "device generator bytes differ (layer %d expert %d)" % (layer, e)
    xd = wl.x[wl.input_index(step), layer].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xd, gen.x(cfg, layer, step)), "device activations differ"


def _run_and_compare(B, cfg, n_steps, samples, tok_sample, hostgen):
    """samples: list of (step, layer) to check."""
    from bench import Workload
    say("[gpu] full-size %s: building workload" % cfg.name)
    wl = Workload(cfg, n_steps, B, DevGen)
    want = set(samples)
    snaps = {}
    for s in range(n_steps):
        if not any(ss == s for ss, _ in want):
            continue
        say("[gpu]   %s: step %d eager, layer by layer" % (cfg.name, s))
        for l in range(cfg.L):
            _run_one_layer(B, wl, s, l)
            if (s, l) in want:
                torch.cuda.synchronize()
                snaps[(s, l)] = _snapshot(wl.buf)
    for (s, l) in samples:
        snap = snaps[(s, l)]
        assert int(snap.status.item()) == 0
        _check_device_generator(wl, cfg, hostgen, l, [0, cfg.E, int(snap.ids[0, 0].item())], step=s)
        say("[gpu]   %s: oracle for step %d layer %d on %d tokens" % (cfg.name, s, l, len(tok_sample)))
        ora, x, wr = _oracle_layer(cfg, hostgen, l, s, tok_sample)
        stats = compare_layer(snap, ora, cfg.T, cfg.k, cfg.E, drawn_logits=cfg.router == "zipf",
                              x64=O.bf16_bits_to_f64(x), w_router=wr)
        say("[gpu]   %s step %d layer %d ok: %s" % (cfg.name, s, l, stats))
    return wl, snaps


def _run_one_layer(B, wl, s, l):
    d, buf = wl.dims, wl.buf
    x = wl.x[wl.input_index(s), l]
    if wl.wr is not None:
        B.moe_route(d, x, wl.wr[l], None, wl.wsg[l], buf.logits, buf.ids, buf.w, buf.sigma)
    else:
        B.moe_route(d, x, None, wl.logits[wl.input_index(s), l], wl.wsg[l], None, buf.ids, buf.w, buf.sigma)
    B.moe_group(d, l, buf.ids, wl.slot_table, wl.n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                buf.status, buf.ws)
    B.moe_expert_ffn(d, x, wl.pool, wl.pool_bytes, wl.layout, buf.offsets, buf.perm, buf.group_slot, buf.h,
                     buf.y_rows, buf.status, buf.ws)
    B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y)


def _one_launch_matches(B, wl, s, l, snap):
    """The same layer through moe_route_group + moe_expert_ffn_combine (gate/up,
    down and combine in one launch) gives the split path's h, Y rows and y bit
    for bit."""
    d, buf = wl.dims, wl.buf
    x = wl.x[wl.input_index(s), l]
    wr = wl.wr[l] if wl.wr is not None else None
    lg = None if wl.wr is not None else wl.logits[wl.input_index(s), l]
    for t in (buf.h, buf.y_rows, buf.y):
        t.fill_(3.0)
    B.moe_route_group(d, l, x, wr, lg, wl.wsg[l], buf.logits if wr is not None else None, buf.ids, buf.w, buf.sigma,
                      wl.slot_table, wl.n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status,
                      buf.ws)
    wl.ffn_combine(x)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == 0
    off_e = int(buf.offsets[wl.cfg.E].item())
    Tk = wl.cfg.T * wl.cfg.k
    live = torch.cat([torch.arange(off_e), torch.arange(Tk, Tk + wl.cfg.T)]).cuda()
    for name in ("h", "y_rows"):
        a, b = getattr(buf, name), getattr(snap, name)
        assert torch.equal(a.view(torch.int16)[live], b.view(torch.int16)[live]), "one launch: %s differs" % name
    assert torch.equal(buf.y.view(torch.int16), snap.y.view(torch.int16)), "one launch: y differs"


def _graph_replays_match_eager(wl, step):
    """Capture one step, replay it 3 times with eager work in between, and check
    each replay's last-layer output against the eager run bit for bit."""
    torch.cuda.synchronize()
    wl.run_step(step)
    torch.cuda.synchronize()
    want = wl.buf.y.view(torch.int16).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.run_step(step)
    for _ in range(3):
        wl.buf.y.zero_()
        wl.run_step(step + 1)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(wl.buf.y.view(torch.int16), want), "graph replay differs from eager"


@pytest.mark.timeout(600)
def test_decode48_full_size(B, hostgen):
    cfg = CONFIGS[2]
    wl, snaps = _run_and_compare(B, cfg, 2, [(0, 0), (0, 23), (0, 47)], list(range(cfg.T)), hostgen)
    say("[gpu]   decode48: one launch (FFN + combine) vs the split path")
    _one_launch_matches(B, wl, 0, 47, snaps[(0, 47)])
    for mode in ("split", "one-launch"):
        say("[gpu]   decode48: graph replay vs eager (%s)" % mode)
        wl.ffn_mode = mode
        _graph_replays_match_eager(wl, 0)
    del wl
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_decode43x64_full_size(B, hostgen):
    cfg = CONFIGS[3]
    wl, snaps = _run_and_compare(B, cfg, 64, [(0, 0), (17, 21), (63, 42)], [0, 7, 15], hostgen)
    say("[gpu]   decode43x64: one launch (FFN + combine) vs the split path")
    _one_launch_matches(B, wl, 63, 42, snaps[(63, 42)])
    del wl
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_prefill8192_full_size(B, hostgen):
    cfg = CONFIGS[4]
    toks = list(range(0, cfg.T, cfg.T // 16)) + [cfg.T - 1]
    wl, _ = _run_and_compare(B, cfg, 1, [(0, 0)], toks, hostgen)
    say("[gpu]   prefill8192: graph replay vs eager")
    _graph_replays_match_eager(wl, 0)
    del wl
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_streamed_ring_matches_resident_and_oracle(B, hostgen):
    """Layers staged through the two-slot ring give bit-identical results to the
    same layers computed from a resident pool ([FreeToken] 3.2: partial results
    merge exactly, bit-identical to a fully resident deployment), and match the
    oracle on sampled tokens."""
    from bench import Workload
    from moe_expert_ffn_top_amd.staged import StagedLayers
    cfg = CONFIGS[5]
    say("[gpu] streamed4x4096: resident reference")
    wl = Workload(cfg, 1, B, DevGen)
    resident = {}
    for l in range(cfg.L):
        _run_one_layer(B, wl, 0, l)
        torch.cuda.synchronize()
        resident[l] = _snapshot(wl.buf)
    say("[gpu] streamed4x4096: pinned host blobs")
    host = torch.empty(wl.pool_bytes, dtype=torch.uint8, pin_memory=True)
    host.copy_(wl.pool)
    torch.cuda.synchronize()
    copy_s, comp_s = torch.cuda.Stream(), torch.cuda.Stream()
    st = StagedLayers(wl.dims, wl.layout, host, cfg.L, copy_s, comp_s)
    staged = {}

    def grab(l):
        comp_s.synchronize()
        staged[l] = _snapshot(st.buf)
    del wl.pool
    torch.cuda.empty_cache()
    say("[gpu] streamed4x4096: staged run")
    with torch.cuda.stream(comp_s):
        st.run(lambda l: wl.x[0, l], lambda l: wl.wsg[l], lambda l: wl.logits[0, l], after_layer=grab)
    torch.cuda.synchronize()
    st.close()
    for l in range(cfg.L):
        assert int(staged[l].status.item()) == 0
        for name in ("ids", "perm", "offsets"):
            assert torch.equal(getattr(staged[l], name), getattr(resident[l], name)), name
        for name in ("h", "y_rows", "y"):
            assert torch.equal(getattr(staged[l], name).view(torch.int16),
                               getattr(resident[l], name).view(torch.int16)), name
    toks = [0, 1000, 2047, 4095]
    for l in (0, 3):
        say("[gpu]   streamed4x4096: oracle layer %d" % l)
        ora, x, wr = _oracle_layer(cfg, hostgen, l, 0, toks)
        stats = compare_layer(staged[l], ora, cfg.T, cfg.k, cfg.E, drawn_logits=True)
        say("[gpu]   streamed4x4096 layer %d ok: %s" % (l, stats))

"""GPU parity at sizes the oracle finishes in seconds (every output compared).

Covers both FFN kernels: the weight-streaming kernel over 16-row tiles (groups
averaging fewer than 16 rows) and the grouped GEMM over 256-row chunks (more).
Covers the tiny workload, several FFN tiles with ragged tails, a reduction
axis that is not a multiple of the 128-value step, reduction axes longer than
4096 (several K rounds per wavefront), GEMM chunks with ragged K steps, column
tiles and row chunks (a group split over two chunks), degenerate shapes (T = 1,
E = k = 1, k = E, E = 1024), a non-resident slot, an out-of-range expert id,
token-permutation invariance and run-to-run determinism."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, bf16_to_f64, compare_layer, say
from oracle import moe_oracle as O
from synth import CONFIGS, Config, HostGen, zipf_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


class Case:
    """Host-generated inputs of one layer (layer 0), uploaded to the GPU."""

    def __init__(self, B, cfg: Config, gen: HostGen, slot_override=None):
        from moe_expert_ffn_top_amd.layer import LayerBuffers
        self.cfg = cfg
        self.dims = B.Dims(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, 1)
        self.layout = B.moe_blob_layout_init(cfg.H, cfg.I)
        olay = O.blob_layout(cfg.H, cfg.I)
        E1 = cfg.E + 1
        self.blobs = {e: gen.expert_blob(cfg, 0, e, olay) for e in range(E1)}
        pool = np.concatenate([self.blobs[e] for e in range(E1)])
        self.pool = torch.from_numpy(pool).cuda()
        self.pool_bytes = pool.nbytes
        st = np.arange(E1, dtype=np.int32)[None, :].copy()
        if slot_override:
            for e, s in slot_override.items():
                st[0, e] = s
        self.slot_table = torch.from_numpy(st).cuda()
        self.x_bits = gen.x(cfg, 0, 0)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        self.wsg = gen.w_shared_gate(cfg, 0)
        self.wsg_t = torch.from_numpy(self.wsg).cuda()
        if cfg.router == "matrix":
            self.wr = gen.w_router(cfg, 0)
            self.wr_t = torch.from_numpy(self.wr).cuda()
            self.logits = None
        else:
            self.wr = None
            self.wr_t = None
            self.logits = zipf_logits(cfg, 0, 0)
            self.logits_t = torch.from_numpy(self.logits).cuda()
        self.buf = LayerBuffers.allocate(self.dims)

    def run(self, B):
        from moe_expert_ffn_top_amd.layer import run_layer
        run_layer(self.buf, 0, self.x, self.pool, self.pool_bytes, self.layout, self.slot_table, self.cfg.E1,
                  self.wsg_t, w_router=self.wr_t, logits=None if self.logits is None else self.logits_t)
        torch.cuda.synchronize()

    def oracle(self, **kw):
        c = self.cfg
        return O.moe_layer(self.x_bits, lambda e: self.blobs[e], c.H, c.I, c.E, c.k, self.wsg,
                           w_router=self.wr, logits=self.logits, **kw)

    def compare(self, ora, **kw):
        return compare_layer(self.buf, ora, self.cfg.T, self.cfg.k, self.cfg.E, drawn_logits=self.logits is not None,
                             x64=O.bf16_bits_to_f64(self.x_bits), w_router=self.wr, **kw)


SMALL = {
    "tiny": CONFIGS[1],
    "multitile_ragged": Config(31, "mt", T=100, H=512, I=256, E=16, k=2, L=1, router="matrix"),
    "ragged_K_zipf": Config(32, "rk", T=37, H=96, I=160, E=10, k=3, L=1, router="zipf", zipf_s=1.0),
    "degenerate_T1_E1": Config(33, "deg", T=1, H=64, I=32, E=1, k=1, L=1, router="matrix"),
    "k_equals_E": Config(34, "kE", T=5, H=128, I=64, E=6, k=6, L=1, router="zipf", zipf_s=0.5),
    "E1024_max": Config(35, "E1024", T=3, H=64, I=64, E=1024, k=8, L=1, router="zipf", zipf_s=1.0),
    "big_k_wide": Config(36, "bk", T=19, H=1024, I=512, E=64, k=16, L=1, router="matrix"),
    # K beyond 4096 on both stages: each wavefront covers its share of K in
    # several rounds, the last one ragged
    "long_K_rounds": Config(37, "lk", T=6, H=4608, I=4352, E=4, k=2, L=1, router="matrix"),
    # grouped-GEMM path: K steps of 64 with a half step at the end (544, 224),
    # column tiles that overhang (224 of 64, 544 of 128), the shared group split
    # over two 256-row chunks
    "gemm_ragged": Config(38, "gr", T=300, H=544, I=224, E=4, k=2, L=1, router="matrix"),
    # GEMM path under Zipf routing: one group above 256 rows, many small ones
    "gemm_zipf_split": Config(39, "gz", T=256, H=256, I=128, E=16, k=4, L=1, router="zipf", zipf_s=1.2),
    # GEMM path with more (chunk, column tile) items than any GPU has CUs: 100
    # chunks give 800 gate/up and 400 down items, so each persistent workgroup
    # walks several, loading the next while finishing the last
    "gemm_many_items": Config(44, "mi", T=2048, H=512, I=512, E=64, k=8, L=1, router="matrix"),
    # small-window routing with T*k above one wavefront's 64 lanes: the sort
    # ranks over 2 (96 entries), 2 with one row in the second (65) and 4 (256)
    # wavefronts
    "sort_f96": Config(45, "s96", T=16, H=256, I=128, E=256, k=6, L=1, router="zipf", zipf_s=1.2),
    "sort_f65": Config(46, "s65", T=13, H=128, I=96, E=40, k=5, L=1, router="zipf", zipf_s=0.7),
    "sort_f256": Config(47, "s256", T=16, H=128, I=64, E=64, k=16, L=1, router="zipf", zipf_s=1.0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(B, hostgen, name):
    cfg = SMALL[name]
    say("[gpu] parity case %s T=%d H=%d I=%d E=%d k=%d" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    case = Case(B, cfg, hostgen)
    case.run(B)
    assert int(case.buf.status.item()) == 0
    stats = case.compare(case.oracle())
    say("[gpu]   %s ok: %s" % (name, stats))


@pytest.mark.parametrize("cname", ["tiny", "k_equals_E", "E1024_max", "big_k_wide", "multitile_ragged",
                                   "decode48_window", "sort_f96", "sort_f65", "sort_f256"])
def test_route_group_matches_separate_calls(B, hostgen, cname):
    """moe_route_group (one fused kernel for T <= 16, T*k <= 256; separate
    kernels otherwise) gives the bits of moe_route then moe_group."""
    cfg = SMALL[cname] if cname in SMALL else Config(40, "dw", T=4, H=2048, I=64, E=512, k=10, L=1, router="zipf",
                                                     zipf_s=1.0)
    say("[gpu] route+group vs separate (%s)" % cname)
    case = Case(B, cfg, hostgen)
    from moe_expert_ffn_top_amd.layer import run_layer
    outs = []
    for fused in (False, True):
        b = case.buf
        for t in (b.ids, b.perm, b.inv_perm, b.offsets, b.group_slot):
            t.fill_(-7)
        b.ws.zero_()
        run_layer(b, 0, case.x, case.pool, case.pool_bytes, case.layout, case.slot_table, cfg.E1, case.wsg_t,
                  w_router=case.wr_t, logits=None if case.logits is None else case.logits_t, fused=fused)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (b.ids, b.w, b.sigma, b.offsets, b.perm, b.inv_perm, b.group_slot,
                                         b.y.view(torch.int16))])
    for u, v in zip(*outs):
        assert torch.equal(u, v)


def test_ffn_stages_split_matches_whole(B, hostgen):
    """gate/up then down as two calls gives the bytes of the single call."""
    cfg = SMALL["multitile_ragged"]
    say("[gpu] FFN stages 1 + 2 vs 3")
    case = Case(B, cfg, hostgen)
    case.run(B)
    b = case.buf
    h_ref, y_ref = b.h.clone(), b.y_rows.clone()
    b.h.zero_()
    b.y_rows.zero_()
    for st in (1, 2):
        B.moe_expert_ffn_stages(case.dims, case.x, case.pool, case.pool_bytes, case.layout, b.offsets, b.perm,
                                b.group_slot, b.h, b.y_rows, b.status, b.ws, st)
    torch.cuda.synchronize()
    assert torch.equal(b.h.view(torch.int16), h_ref.view(torch.int16))
    assert torch.equal(b.y_rows.view(torch.int16), y_ref.view(torch.int16))


@pytest.mark.parametrize("cname", ["tiny", "gemm_ragged"])
def test_non_resident_slot_gives_zero_rows_and_status(B, hostgen, cname):
    cfg = CONFIGS[1] if cname == "tiny" else SMALL[cname]
    say("[gpu] non-resident slot case (%s)" % cname)
    probe = Case(B, cfg, hostgen)
    probe.run(B)
    ids = probe.buf.ids.cpu().numpy()
    missing = int(ids[0, 0])            # an expert that token 0 picks
    case = Case(B, cfg, hostgen, slot_override={missing: -1})
    case.run(B)
    assert int(case.buf.status.item()) & B.MOE_DEV_NOT_RESIDENT
    ora = case.oracle()
    inv = case.buf.inv_perm.cpu().numpy()
    T, k = cfg.T, cfg.k
    yr = np.zeros((T, k, cfg.H))
    for t in range(T):
        for j in range(k):
            if ora.ids[t, j] != missing:
                yr[t, j] = ora.y_rows[int(ora.groups.inv_perm[t * k + j])]
    ysh = np.stack([ora.y_rows[T * k + t] for t in range(T)])
    y_ref, _ = O.combine(yr, ora.w, ora.sigma, ysh)
    rows = [int(inv[t * k + j]) for t in range(T) for j in range(k) if ids[t, j] == missing]
    assert rows and np.all(bf16_to_f64(case.buf.y_rows[rows]) == 0)
    assert np.all(bf16_to_f64(case.buf.h[rows]) == 0)
    assert_close(bf16_to_f64(case.buf.y), y_ref, "y with a non-resident expert")


def test_bad_expert_id_is_dropped_and_flagged(B, hostgen):
    cfg = CONFIGS[1]
    say("[gpu] bad expert id case")
    case = Case(B, cfg, hostgen)
    case.run(B)
    ora = case.oracle()
    d, buf = case.dims, case.buf
    ids = buf.ids.clone()
    ids[2, 1] = cfg.E            # out of range
    buf.status.zero_()
    B.moe_group(d, 0, ids, case.slot_table, cfg.E1, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                buf.status, buf.ws)
    B.moe_expert_ffn(d, case.x, case.pool, case.pool_bytes, case.layout, buf.offsets, buf.perm, buf.group_slot,
                     buf.h, buf.y_rows, buf.status, buf.ws)
    B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y)
    torch.cuda.synchronize()
    assert int(buf.status.item()) & B.MOE_DEV_BAD_EXPERT_ID
    assert int(buf.inv_perm[2 * cfg.k + 1].item()) == -1
    off = buf.offsets.cpu().numpy()
    assert off[cfg.E] == cfg.T * cfg.k - 1 and off[cfg.E + 1] == cfg.T * cfg.k + cfg.T
    T, k = cfg.T, cfg.k
    yr = np.stack([np.stack([ora.y_rows[int(ora.groups.inv_perm[t * k + j])] for j in range(k)]) for t in range(T)])
    yr[2, 1] = 0.0
    ysh = np.stack([ora.y_rows[T * k + t] for t in range(T)])
    y_ref, _ = O.combine(yr, ora.w, ora.sigma, ysh)
    assert_close(bf16_to_f64(buf.y), y_ref, "y with a dropped id")


@pytest.mark.parametrize("cname", ["multitile_ragged", "gemm_ragged"])
def test_token_permutation_bit_exact_on_gpu(B, hostgen, cname):
    cfg = SMALL[cname]
    say("[gpu] token permutation case (%s)" % cname)
    a = Case(B, cfg, hostgen)
    a.run(B)
    pi = np.random.default_rng(7).permutation(cfg.T)
    b = Case(B, cfg, hostgen)
    b.x_bits = a.x_bits[pi]
    b.x = torch.from_numpy(b.x_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    b.run(B)
    pi_t = torch.as_tensor(pi, device="cuda")
    assert torch.equal(b.buf.ids, a.buf.ids[pi_t])
    assert torch.equal(b.buf.y.view(torch.int16), a.buf.y.view(torch.int16)[pi_t])


@pytest.mark.parametrize("cname", ["multitile_ragged", "gemm_ragged"])
def test_run_to_run_determinism(B, hostgen, cname):
    cfg = SMALL[cname]
    say("[gpu] determinism case (%s)" % cname)
    a = Case(B, cfg, hostgen)
    a.run(B)
    first = [t.clone() for t in (a.buf.ids, a.buf.perm, a.buf.h.view(torch.int16), a.buf.y.view(torch.int16))]
    for _ in range(3):
        a.run(B)
        again = (a.buf.ids, a.buf.perm, a.buf.h.view(torch.int16), a.buf.y.view(torch.int16))
        for u, v in zip(first, again):
            assert torch.equal(u, v)


def _drawn_ids(rng, T, k, E, zipf_s):
    """k distinct experts per token: Gumbel top-k over log-weights
    -zipf_s * log(rank) (zipf_s = 0: uniform)."""
    logw = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    keys = logw[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


# (T, k, E, zipf_s): the prefill shapes (512 and 256 experts, one int4 of four
# experts per count load), E = 1024, and E not a multiple of 4 (one expert per
# load) with enough 256-entry blocks that every scan thread runs full batches
@pytest.mark.parametrize("T,k,E,zs", [(8192, 10, 512, 0.0), (4096, 6, 256, 1.2), (600, 8, 1024, 1.0),
                                      (100000, 3, 10, 0.5), (97, 3, 7, 0.0)])
def test_group_matches_oracle_on_drawn_ids(B, T, k, E, zs):
    """moe_group on drawn ids gives the oracle's offsets, perm and inv_perm bit
    for bit, and the slot table's entries as group slots, whichever of its
    kernel paths the size selects."""
    from moe_expert_ffn_top_amd.layer import LayerBuffers
    say("[gpu] grouping case T=%d k=%d E=%d zipf=%.1f" % (T, k, E, zs))
    ids = _drawn_ids(np.random.default_rng(T * 31 + E), T, k, E, zs)
    d = B.Dims(T, 64, 32, E, k, 1)
    buf = LayerBuffers.allocate(d)
    buf.ids.copy_(torch.from_numpy(ids))
    st = torch.from_numpy((np.arange(E + 1, dtype=np.int32)[::-1] + 3)[None, :].copy()).cuda()
    buf.status.zero_()
    B.moe_group(d, 0, buf.ids, st, E + 4, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status, buf.ws)
    torch.cuda.synchronize()
    g = O.group(ids, E)
    assert int(buf.status.item()) == 0
    assert np.array_equal(buf.offsets.cpu().numpy(), g.offsets)
    assert np.array_equal(buf.perm.cpu().numpy(), g.perm)
    assert np.array_equal(buf.inv_perm.cpu().numpy(), g.inv_perm)
    assert np.array_equal(buf.group_slot.cpu().numpy(), st.cpu().numpy()[0])


# (T, E, k): the radix select with 8, 2 and 16 keys per lane, k above 64 (two
# entries per lane to rank), k above 128 (the one-winner-per-round path), and
# the fused decode kernel (T <= 16, T k <= 256)
# (4, 512, 10), (3, 1024, 8), (2, 300, 16) and (8, 128, 4) run moe_route_group's
# top-k over several wavefronts per token (merged by rank; 300 experts split in
# parts of 75, 16 x 4 candidates filling one wavefront)
@pytest.mark.parametrize("T,E,k", [(64, 512, 10), (40, 100, 70), (8, 512, 200), (4, 512, 10), (16, 256, 6),
                                   (33, 1024, 8), (3, 1024, 8), (2, 300, 16), (8, 128, 4)])
def test_topk_with_ties_matches_oracle(B, T, E, k):
    """Drawn logits on a half-unit grid tie everywhere; the winners and their
    slot order (logit descending, lower expert index first among equal
    logits, -0 equal to +0) match the oracle's top-k exactly, and the weights
    match its softmax."""
    from moe_expert_ffn_top_amd.layer import LayerBuffers
    say("[gpu] top-k ties case T=%d E=%d k=%d" % (T, E, k))
    rng = np.random.default_rng(T * 7 + E + k)
    lg = (np.round(rng.normal(size=(T, E)) * 2) / 2).astype(np.float32)
    lg[0, :] = 0.25                       # one value everywhere
    if T > 1:
        lg[1, 0::2] = -0.0                # the two zeros tie
        lg[1, 1::2] = 0.0
    want_ids = O.topk(lg, k)
    want_w = O.topk_weights(lg, want_ids)
    d = B.Dims(T, 64, 32, E, k, 1)
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device="cuda")
    wsg = torch.zeros(64, dtype=torch.float32, device="cuda")
    lg_t = torch.from_numpy(lg).cuda()
    buf = LayerBuffers.allocate(d)
    B.moe_route(d, x, None, lg_t, wsg, None, buf.ids, buf.w, buf.sigma)
    torch.cuda.synchronize()
    assert np.array_equal(buf.ids.cpu().numpy(), want_ids)
    assert np.max(np.abs(buf.w.cpu().numpy().astype(np.float64) - want_w)) <= 1e-6
    if T <= 16 and T * k <= 256:
        st = torch.arange(E + 1, dtype=torch.int32, device="cuda").view(1, E + 1).contiguous()
        buf.ids.fill_(-7)
        buf.status.zero_()
        B.moe_route_group(d, 0, x, None, lg_t, wsg, None, buf.ids, buf.w, buf.sigma, st, E + 1, buf.offsets,
                          buf.perm, buf.inv_perm, buf.group_slot, buf.status, buf.ws)
        torch.cuda.synchronize()
        assert np.array_equal(buf.ids.cpu().numpy(), want_ids)
        assert np.max(np.abs(buf.w.cpu().numpy().astype(np.float64) - want_w)) <= 1e-6
        assert int(buf.status.item()) == 0
        g = O.group(want_ids, E)
        assert np.array_equal(buf.perm.cpu().numpy(), g.perm)
        assert np.array_equal(buf.inv_perm.cpu().numpy(), g.inv_perm)
        assert np.array_equal(buf.offsets.cpu().numpy(), g.offsets)


def _late_logits(T, E, k, late, seed):
    """Drawn logits in which each expert of `late` is picked, when at all, only
    at the last slot k - 1 (every other token leaves it unpicked)."""
    rng = np.random.default_rng(seed)
    lg = rng.normal(size=(T, E)).astype(np.float32)
    lg[:, late] = -20.0
    for t in range(0, T, 2):
        others = np.sort(np.delete(lg[t], late))[::-1]
        lg[t, late[(t // 2) % len(late)]] = (others[k - 2] + others[k - 1]) / 2
    return lg


# one decode-sized window (single-kernel grouping) and one large window
# (multi-kernel grouping, grouped-GEMM FFN)
TAIL = {
    "window12": Config(41, "ts", T=12, H=128, I=64, E=12, k=3, L=1, router="zipf", zipf_s=1.0),
    "window300": Config(42, "tl", T=300, H=128, I=64, E=12, k=3, L=1, router="zipf", zipf_s=1.0),
}


@pytest.mark.parametrize("cname", list(TAIL))
def test_tail_skip_matches_oracle(B, hostgen, cname):
    """moe_group_tail_skip: non-resident experts that every token of the window
    ranks at the threshold or later are skipped (zero rows, no renormalisation,
    MOE_DEV_TAIL_SKIPPED, counted); a non-resident expert some token ranks
    earlier still sets MOE_DEV_NOT_RESIDENT; threshold 0 skips nothing."""
    cfg = TAIL[cname]
    T, k, E = cfg.T, cfg.k, cfg.E
    late = [9, 10, 11]
    say("[gpu] tail-skip case %s T=%d E=%d k=%d" % (cname, T, E, k))
    case = Case(B, cfg, hostgen, slot_override={e: -1 for e in late})
    case.logits = _late_logits(T, E, k, late, cfg.cfg_id)
    case.logits_t = torch.from_numpy(case.logits).cuda()
    d, buf = case.dims, case.buf
    ns = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def run(R, slot_table):
        B.moe_route(d, case.x, None, case.logits_t, case.wsg_t, None, buf.ids, buf.w, buf.sigma)
        buf.status.zero_()
        B.moe_group_tail_skip(d, 0, buf.ids, slot_table, cfg.E1, R, buf.offsets, buf.perm, buf.inv_perm,
                              buf.group_slot, buf.status, ns, buf.ws)
        B.moe_expert_ffn(d, case.x, case.pool, case.pool_bytes, case.layout, buf.offsets, buf.perm, buf.group_slot,
                         buf.h, buf.y_rows, buf.status, buf.ws)
        B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y)
        torch.cuda.synchronize()
        return int(buf.status.item()), int(ns.item())

    resident = np.ones(E, bool)
    resident[late] = False
    status, n = run(k - 1, case.slot_table)
    ora_ids = O.topk(case.logits, k)
    assert np.array_equal(buf.ids.cpu().numpy(), ora_ids)
    mask = O.tail_skip(ora_ids, resident, k - 1)
    assert list(np.nonzero(mask)[0]) == late
    assert status == B.MOE_DEV_TAIL_SKIPPED and n == len(late)
    ora = case.oracle(skip=mask)
    inv = buf.inv_perm.cpu().numpy()
    rows = [int(inv[t * k + j]) for t in range(T) for j in range(k) if mask[ora_ids[t, j]]]
    assert rows and np.all(bf16_to_f64(buf.y_rows[rows]) == 0)
    assert_close(bf16_to_f64(buf.y), ora.y_pre, "y with tail-skip")

    # a non-resident expert that a token ranks first is not skippable
    first = int(ora_ids[1, 0])
    st2 = case.slot_table.clone()
    st2[0, first] = -1
    status, n = run(k - 1, st2)
    assert status == B.MOE_DEV_TAIL_SKIPPED | B.MOE_DEV_NOT_RESIDENT and n == len(late)
    # threshold 0: no skipping
    status, n = run(0, case.slot_table)
    assert status == B.MOE_DEV_NOT_RESIDENT and n == 0

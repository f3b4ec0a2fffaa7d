"""GPU parity of the MX variant: MXFP4 experts, MXFP8 activations, scaled MFMA.

- MXFP8 quantisation (moe_quantize_mxfp8): codes and scales bit for bit
  against the oracle, on values that span the E8M0 range, zero blocks, bf16
  subnormals, saturation and E4M3 ties.
- Whole layers through moe_expert_ffn_mx against oracle.moe_layer(fmt="mx"),
  nothing of the kernel fed to the oracle: ids and groups bit-exact; h bit for
  bit but for R1 near ties (resolve_h_near_ties: the oracle's exact h_pre at a
  bf16 rounding boundary, within the kernel's fp32 error, where either
  rounding is valid; the oracle then carries the kernel's choice on to Y and
  y); Y rows and y to the float bar of gpu_util.  The workspace's quantised x
  and h are also checked bit for bit against the oracle's quantisation of the
  same bf16 values (x, and the kernel's own h).
- Why h can be held bit for bit: the grouped GEMM's gate/up issues the split
  pair of scaled MFMAs (split_e4m3), so g and u are exact up to fp32 addition
  (tests/test_gpu_probes.py pins the instruction's truncation and the split);
  the decode kernel runs bf16 MFMAs on exactly decoded values.
- Edge cases:
  - a one-step K (I = 128);
  - an odd step count (H = 384);
  - groups over two 256-row chunks and ragged tails;
  - more items than workgroups;
  - a non-resident group;
  - stages split;
  - the device pool generator against the host one.
- Decode-sized groups (T k < 16 E): the weight-streaming kernel on MX blobs,
  its A rows the bf16 values of MXFP8(x) and MXFP8(h), both bit for bit
  against the oracle's quantisation; a K split into several rounds (H = 4608).
- Full size: decode48_mx on all four tokens of its last layer, prefill8192_mx
  on 17 sampled tokens.
- moe_route_group_ffn_mx (route, group and MXFP8(x) in one launch for decode
  windows) against moe_route_group then moe_expert_ffn_mx, every output bit
  for bit, on the decode48 window, T k = 96 and 65, the router matrix, and a
  prefill shape (separate kernels)."""
import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say, bf16_to_f64
from oracle import moe_oracle as O
from synth import CONFIGS, Config, HostGen, DevGen, zipf_logits

pytestmark = pytest.mark.gpu


# The kernel's g and u are fp32 sums of exactly computed block sums (the split
# MFMA of the grouped GEMM, bf16 MFMAs on exact values in the decode kernel),
# so each lies within a few fp32 rounding errors of sum |products| of the
# exact sum; NEAR_TIE_EPS bounds that: 2^-22 of sum |products|, 4 times the
# rounding unit of that sum.  (Measured: every flip of the split kernel lies
# within the epilogue's own fp32 error of the boundary; the single-MFMA
# kernel's flips need up to 2^-18.8, hundreds of them more than 2^-20.)
NEAR_TIE_EPS = 2.0 ** -22


def _bf16_key(v):
    """An integer that steps by one between adjacent bf16 values (v bf16-exact)."""
    bits = (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.int64)
    return np.where(bits & 0x8000, -(bits & 0x7FFF), bits)


def resolve_h_near_ties(buf, ora, cfg, blob_of, x64):
    """The oracle's result, with h taken from the kernel at each R1 near tie.

    h = bf16(silu(g) u) decides the MXFP8 codes of h (RA) downstream, so an
    element whose exact pre-rounding value h_pre lies at a bf16 rounding
    boundary can round either way within fp32 accuracy, and each way is a
    valid result.  Every h element of the compared rows must equal the
    oracle's bit for bit, except where (a) the kernel's value is the other bf16
    neighbour of the oracle's and (b) the oracle's own h_pre lies within what
    the kernel's fp32 error can move it of the boundary between the two: g and u
    each off by at most NEAR_TIE_EPS * sum |products| (from the oracle's MXFP8
    of x and its MX weights), silu's slope at most 1.1, and the epilogue's
    fp32 exp, reciprocal and products.  Only there the kernel's value is
    adopted, and the oracle recomputes that row's Y (down_mx) and the outputs y
    (combine).  Returns (result, number adopted, largest distance / window)."""
    import copy
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    olay = O.mx_blob_layout(H, I)
    same_tok = np.all(buf.ids.cpu().numpy() == ora.ids, axis=1)
    perm, off = ora.groups.perm, ora.groups.offsets

    def owner(p):   # (expert, token) of row p
        if p >= T * k:
            return E, p - T * k
        return int(np.searchsorted(off[:E + 1], p, side="right") - 1), int(perm[p]) // k

    rows = sorted(p for p in ora.h if same_tok[owner(p)[1]])
    if not rows:
        return ora, 0, 0.0
    hk = bf16_to_f64(buf.h.index_select(0, torch.as_tensor(rows, device=buf.h.device)))
    ho = np.stack([ora.h[p] for p in rows])
    bad = np.argwhere(hk != ho)
    if bad.size == 0:
        return ora, 0, 0.0
    new = copy.copy(ora)
    new.h, new.y_rows, new.y_rows_pre = dict(ora.h), dict(ora.y_rows), dict(ora.y_rows_pre)
    weights, gu = {}, {}
    worst = 0.0
    adopted = {}
    for i, j in bad:
        p = rows[i]
        e, t = owner(p)
        if e not in weights:
            weights[e] = tuple(O.mx_dequant(blob_of(e), olay, m, H, I) for m in range(3))
        if p not in gu:
            xq = O.mxfp8_quantize(x64[t][None])[2][0]
            wg, wu, _ = weights[e]
            gu[p] = (xq @ wg.T, np.abs(xq) @ np.abs(wg).T, xq @ wu.T, np.abs(xq) @ np.abs(wu).T)
        g, sg, u, su = (v[j] for v in gu[p])
        hp = ora.h_pre[p][j]
        assert abs(int(_bf16_key(hk[i, j])) - int(_bf16_key(ho[i, j]))) == 1, (
            "h row %d unit %d: %r is not a bf16 neighbour of the oracle's %r" % (p, j, hk[i, j], ho[i, j]))
        dg, du = NEAR_TIE_EPS * sg, NEAR_TIE_EPS * su
        sil = g / (1.0 + np.exp(-g))
        window = (1.1 * dg * (abs(u) + du) + (abs(sil) + 1.1 * dg) * du
                  + (1.5 * abs(g) + 8.0) * 2.0 ** -24 * abs(hp))
        dist = abs(hp - 0.5 * (hk[i, j] + ho[i, j]))
        assert dist <= window, ("h row %d unit %d differs from the oracle's (%r vs %r) and is no R1 near tie: "
                                "h_pre %r lies %.3e from the rounding boundary, window %.3e" % (
                                    p, j, hk[i, j], ho[i, j], hp, dist, window))
        worst = max(worst, dist / window)
        adopted.setdefault(p, []).append((i, j))
    for p, ij in adopted.items():
        e, _ = owner(p)
        hr = ora.h[p].copy()
        for i, j in ij:
            hr[j] = hk[i, j]
        new.h[p] = hr
        y_pre, y = O.down_mx(hr[None], weights[e][2])
        new.y_rows_pre[p], new.y_rows[p] = y_pre[0], y[0]
    inv = ora.groups.inv_perm
    tok = [int(t) for t in ora.tokens]
    yr = np.stack([np.stack([new.y_rows[int(inv[t * k + j])] for j in range(k)]) for t in tok])
    ysh = np.stack([new.y_rows[T * k + t] for t in tok])
    new.y_pre, new.y = O.combine(yr, ora.w[tok], ora.sigma[tok], ysh)
    return new, int(len(bad)), float(worst)


def end_to_end_y(buf, ora):
    """The kernel's y against the oracle's own chain, for the log: relative L2
    and the largest element error as a multiple of rms (the bar itself is
    asserted by compare_layer)."""
    tok = [int(t) for t in ora.tokens]
    y = bf16_to_f64(buf.y.index_select(0, torch.as_tensor(tok, device=buf.y.device)))
    d = y - ora.y_pre
    rel = float(np.linalg.norm(d) / np.linalg.norm(ora.y_pre))
    return dict(rel_l2=rel, max_over_rms=float(np.abs(d).max() / np.sqrt(np.mean(ora.y_pre ** 2))))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


class MxCase:
    """Host-generated MX inputs of one layer (layer 0), uploaded to the GPU."""

    def __init__(self, B, cfg: Config, gen: HostGen, slot_override=None):
        from moe_expert_ffn_top_amd.layer import LayerBuffers
        self.cfg = cfg
        self.dims = B.Dims(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, 1)
        self.layout = B.moe_blob_layout_init_mx(cfg.H, cfg.I)
        olay = O.mx_blob_layout(cfg.H, cfg.I)
        E1 = cfg.E + 1
        self.blobs = {e: gen.expert_blob_mx(cfg, 0, e, olay) for e in range(E1)}
        pool = np.concatenate([self.blobs[e] for e in range(E1)])
        self.pool = torch.from_numpy(pool).cuda()
        self.pool_bytes = pool.nbytes
        st = np.arange(E1, dtype=np.int32)[None, :].copy()
        for e, s in (slot_override or {}).items():
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
            self.wr, self.wr_t = None, None
            self.logits = zipf_logits(cfg, 0, 0)
            self.logits_t = torch.from_numpy(self.logits).cuda()
        self.buf = LayerBuffers.allocate(self.dims, mx=True)
        self.mws = B.MxWorkspace(self.dims)

    def run(self, B):
        from moe_expert_ffn_top_amd.layer import run_layer
        self.buf.status.zero_()
        run_layer(self.buf, 0, self.x, self.pool, self.pool_bytes, self.layout, self.slot_table, self.cfg.E1,
                  self.wsg_t, w_router=self.wr_t, logits=None if self.logits is None else self.logits_t)
        torch.cuda.synchronize()

    def oracle(self, **kw):
        c = self.cfg
        return O.moe_layer(self.x_bits, lambda e: self.blobs[e], c.H, c.I, c.E, c.k, self.wsg, w_router=self.wr,
                           logits=self.logits, fmt="mx", **kw)

    def compare(self, ora):
        """Against the oracle's own chain: h bit for bit but for R1 near ties
        (resolve_h_near_ties), then compare_layer's bar on h, Y and y."""
        kw = dict(drawn_logits=self.logits is not None, x64=O.bf16_bits_to_f64(self.x_bits), w_router=self.wr)
        res, ties, worst = resolve_h_near_ties(self.buf, ora, self.cfg, lambda e: self.blobs[e], kw["x64"])
        say("[gpu]   h near ties adopted: %d (largest distance %.2f of its window)" % (ties, worst))
        say("[gpu]   end to end: %s" % end_to_end_y(self.buf, ora))
        stats = compare_layer(self.buf, res, self.cfg.T, self.cfg.k, self.cfg.E, **kw)
        stats["h_near_ties"] = ties
        return stats

    def ws_section(self, off, n):
        return self.buf.mx_ws[off:off + n].cpu().numpy()

    def check_quantised_workspace(self, rows=None):
        """xq/xs and hq/hs (or, for decode shapes, the bf16 values xb/hb) against
        the oracle's MXFP8 of x and of the kernel's h."""
        c, m = self.cfg, self.mws
        if not m.gemm:
            nr = c.T * c.k + c.T
            xb = self.buf.mx_ws[m.off_xb:m.off_xb + c.T * c.H * 2].view(torch.bfloat16).view(c.T, c.H)
            assert np.array_equal(bf16_to_f64(xb), O.mxfp8_quantize(O.bf16_bits_to_f64(self.x_bits))[2]), "x values"
            hb = self.buf.mx_ws[m.off_hb:m.off_hb + nr * c.I * 2].view(torch.bfloat16).view(nr, c.I)
            # rows of groups that exist (rows past offsets[E] of dropped entries are not written)
            off = self.buf.offsets.cpu().numpy()
            live = np.r_[np.arange(int(off[c.E])), np.arange(c.T * c.k, nr)]
            want = O.mxfp8_quantize(bf16_to_f64(self.buf.h)[live])[2]
            assert np.array_equal(bf16_to_f64(hb)[live], want), "h values"
            return
        xc, xs, _ = O.mxfp8_quantize(O.bf16_bits_to_f64(self.x_bits))
        assert np.array_equal(self.ws_section(m.off_xq, c.T * c.H).reshape(c.T, c.H), xc), "x codes"
        gxs = self.ws_section(m.off_xs, c.T * m.xs_stride).reshape(c.T, m.xs_stride)[:, :c.H // 32]
        assert np.array_equal(gxs, xs), "x scales"
        nr = c.T * c.k + c.T
        h = bf16_to_f64(self.buf.h)
        hc, hs, _ = O.mxfp8_quantize(h)
        gq = self.ws_section(m.off_hq, nr * c.I).reshape(nr, c.I)
        gs = self.ws_section(m.off_hs, nr * m.hs_stride).reshape(nr, m.hs_stride)[:, :c.I // 32]
        rows = np.arange(nr) if rows is None else np.asarray(rows)
        bad = np.nonzero(np.any(gq[rows] != hc[rows], axis=1) | np.any(gs[rows] != hs[rows], axis=1))[0]
        assert bad.size == 0, "h codes/scales differ on %d rows, first %s" % (bad.size, rows[bad[:5]])


MX_SMALL = {
    # one group per expert of ~16 rows; down is a single K step (I = 128)
    "mx_small": Config(51, "mxs", T=64, H=256, I=128, E=8, k=2, L=1, router="matrix", fmt="mx"),
    # groups over two 256-row chunks with ragged tails; the shared group over 3 chunks
    "mx_multichunk": Config(52, "mxm", T=700, H=512, I=256, E=4, k=2, L=1, router="matrix", fmt="mx"),
    # Zipf routing: one group above 256 rows and many small ones; H = 384 (3 K steps)
    "mx_zipf": Config(53, "mxz", T=256, H=384, I=128, E=16, k=4, L=1, router="zipf", zipf_s=1.2, fmt="mx"),
    # more (chunk, column tile) items than CUs (100 chunks: 800 gate/up and
    # 400 down items), so each persistent workgroup walks several
    "mx_many_items": Config(54, "mxi", T=2048, H=512, I=512, E=64, k=8, L=1, router="matrix", fmt="mx"),
}


MX_DEC = {
    # a decode window under Zipf routing
    "mxd_small": Config(61, "mxd", T=4, H=256, I=128, E=32, k=4, L=1, router="zipf", zipf_s=1.0, fmt="mx"),
    # 16 tokens through the router matrix; several unit blocks per item
    "mxd_multi": Config(62, "mxdm", T=16, H=512, I=256, E=64, k=6, L=1, router="matrix", fmt="mx"),
    # K split over wavefronts and covered in several rounds, the last ragged
    "mxd_longK": Config(63, "mxdl", T=6, H=4608, I=1152, E=8, k=2, L=1, router="matrix", fmt="mx"),
}


@pytest.mark.parametrize("name", list(MX_DEC))
def test_mx_decode_layer_parity(B, hostgen, name):
    cfg = MX_DEC[name]
    assert cfg.T * cfg.k < 16 * cfg.E
    say("[gpu] mx decode-path parity %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = MxCase(B, cfg, hostgen)
    assert not c.mws.gemm
    c.run(B)
    assert int(c.buf.status.item()) == 0
    c.check_quantised_workspace()
    stats = c.compare(c.oracle())
    say("[gpu]   %s: %s" % (name, stats))


def test_mx_decode_non_resident_group(B, hostgen):
    cfg = MX_DEC["mxd_multi"]
    say("[gpu] mx decode non-resident group")
    c = MxCase(B, cfg, hostgen)
    c.run(B)
    off = c.buf.offsets.cpu().numpy()
    e = int(np.argmax(np.diff(off[:cfg.E + 1])))   # an expert with rows
    d = MxCase(B, cfg, hostgen, slot_override={e: -1})
    d.run(B)
    assert int(d.buf.status.item()) & B.MOE_DEV_NOT_RESIDENT
    assert torch.count_nonzero(d.buf.y_rows[off[e]:off[e + 1]].float()) == 0
    keep = torch.ones(cfg.T * cfg.k + cfg.T, dtype=torch.bool, device="cuda")
    keep[off[e]:off[e + 1]] = False
    assert torch.equal(d.buf.y_rows[keep].view(torch.int16), c.buf.y_rows[keep].view(torch.int16))


def test_quantize_mxfp8_bit_exact(B):
    say("[gpu] mx: MXFP8 quantisation vs oracle")
    rng = np.random.default_rng(17)
    rows, K = 41, 2048
    v = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-40, 40, (rows, 1)))
    v *= np.exp2(rng.uniform(-12, 0, v.shape))               # wide range inside each block
    v[0] = 0.0                                               # zero row: scale byte 0, codes 0
    v[1, :32] = -0.0                                         # negative zeros
    v[2] = rng.standard_normal(K) * 2.0 ** -130              # bf16 subnormals
    v[3] = rng.standard_normal(K) * 2.0 ** 120               # near the top of the range
    v[4] = 511.0                                             # saturates (X = 1): 448
    # exact E4M3 ties: amax 256 (X = 1), odd multiples of half a step
    v[5] = np.tile(np.array([256.0] + [1.0625, 1.1875, 17.0, 19.0, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9] * 5 + [3.0]), K // 32)
    bits = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    xb = bits.view(torch.int16).numpy().view(np.uint16)
    x = bits.cuda()
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(x, rows, K, codes, scales)
    torch.cuda.synchronize()
    oc, os_, _ = O.mxfp8_quantize(O.bf16_bits_to_f64(xb))
    assert np.array_equal(scales.cpu().numpy(), os_), "scales"
    gc = codes.cpu().numpy()
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, "codes differ at %s (gpu %s oracle %s)" % (bad[:5].tolist(), gc[tuple(bad[0])],
                                                                     oc[tuple(bad[0])])


@pytest.mark.parametrize("name", list(MX_SMALL))
def test_mx_layer_parity(B, hostgen, name):
    cfg = MX_SMALL[name]
    say("[gpu] mx layer parity %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = MxCase(B, cfg, hostgen)
    c.run(B)
    assert int(c.buf.status.item()) == 0
    c.check_quantised_workspace()
    stats = c.compare(c.oracle())
    say("[gpu]   %s: %s" % (name, stats))


def test_mx_non_resident_group_gives_zero_rows(B, hostgen):
    cfg = MX_SMALL["mx_small"]
    say("[gpu] mx non-resident group")
    c = MxCase(B, cfg, hostgen, slot_override={3: -1})
    c.run(B)
    assert int(c.buf.status.item()) & B.MOE_DEV_NOT_RESIDENT
    off = c.buf.offsets.cpu().numpy()
    assert off[4] > off[3], "expert 3 has rows"
    h = c.buf.h[off[3]:off[4]].float()
    y = c.buf.y_rows[off[3]:off[4]].float()
    assert torch.count_nonzero(h) == 0 and torch.count_nonzero(y) == 0
    # the other groups are unaffected
    full = MxCase(B, cfg, hostgen)
    full.run(B)
    keep = torch.ones(cfg.T * cfg.k + cfg.T, dtype=torch.bool, device="cuda")
    keep[off[3]:off[4]] = False
    assert torch.equal(c.buf.y_rows[keep].view(torch.int16), full.buf.y_rows[keep].view(torch.int16))


def test_mx_stages_split_matches_whole(B, hostgen):
    cfg = MX_SMALL["mx_multichunk"]
    say("[gpu] mx stages split")
    c = MxCase(B, cfg, hostgen)
    c.run(B)
    want = c.buf.y_rows.view(torch.int16).clone()
    c.buf.y_rows.zero_()
    d, buf = c.dims, c.buf
    for st in (1, 2):
        B.moe_expert_ffn_mx(d, c.x, c.pool, c.pool_bytes, c.layout, buf.offsets, buf.perm, buf.group_slot, buf.h,
                            buf.y_rows, buf.status, buf.ws, buf.mx_ws, st)
    torch.cuda.synchronize()
    assert torch.equal(buf.y_rows.view(torch.int16), want)


def test_device_mx_pool_matches_host(B, hostgen):
    cfg = MX_SMALL["mx_zipf"]
    say("[gpu] mx device pool generator vs host")
    lay = B.moe_blob_layout_init_mx(cfg.H, cfg.I)
    olay = O.mx_blob_layout(cfg.H, cfg.I)
    E1 = cfg.E1
    table = torch.arange(E1, dtype=torch.int32, device="cuda").view(1, E1).contiguous()
    pool = torch.zeros(E1 * lay.slot_stride, dtype=torch.uint8, device="cuda")
    DevGen().pool_mx(cfg, 0, 1, table.data_ptr(), E1, lay, pool.data_ptr())
    torch.cuda.synchronize()
    got = pool.view(E1, lay.slot_stride).cpu().numpy()
    for e in range(E1):
        assert np.array_equal(got[e], hostgen.expert_blob_mx(cfg, 0, e, olay)), "expert %d" % e


@pytest.mark.timeout(600)
def test_decode48_mx_full_size(B, hostgen):
    """A whole 48-layer decode step on MX blobs; the buffers then hold layer 47,
    checked against the oracle on all four tokens."""
    from bench import Workload
    cfg = CONFIGS[8]
    say("[gpu] full-size %s: building workload" % cfg.name)
    wl = Workload(cfg, 1, B, DevGen)
    wl.run_step(0)
    torch.cuda.synchronize()
    buf, l = wl.buf, cfg.L - 1
    assert int(buf.status.item()) == 0
    olay = O.mx_blob_layout(cfg.H, cfg.I)
    x = hostgen.x(cfg, l, 0)
    lg = zipf_logits(cfg, l, 0)
    need = set(O.topk(lg, cfg.k).reshape(-1).tolist()) | {cfg.E}
    blobs = {e: hostgen.expert_blob_mx(cfg, l, e, olay) for e in need}
    stride = wl.layout.slot_stride
    s0 = l * cfg.E1 + cfg.E
    assert np.array_equal(wl.pool[s0 * stride:s0 * stride + olay.blob_bytes].cpu().numpy(),
                          blobs[cfg.E][:olay.blob_bytes]), "device pool bytes"
    say("[gpu]   %s: oracle for layer %d" % (cfg.name, l))
    ora = O.moe_layer(x, lambda e: blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, hostgen.w_shared_gate(cfg, l), logits=lg,
                      fmt="mx")
    res, ties, worst = resolve_h_near_ties(buf, ora, cfg, lambda e: blobs[e], O.bf16_bits_to_f64(x))
    say("[gpu]   h near ties adopted: %d (largest distance %.2f of its window)" % (ties, worst))
    say("[gpu]   end to end: %s" % end_to_end_y(buf, ora))
    stats = compare_layer(buf, res, cfg.T, cfg.k, cfg.E, drawn_logits=True)
    say("[gpu]   %s ok: %s" % (cfg.name, stats))
    del wl
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_prefill8192_mx_full_size(B, hostgen):
    from bench import Workload
    cfg = CONFIGS[7]
    say("[gpu] full-size %s: building workload" % cfg.name)
    wl = Workload(cfg, 1, B, DevGen)
    wl.run_step(0)
    torch.cuda.synchronize()
    buf = wl.buf
    assert int(buf.status.item()) == 0
    toks = list(range(0, cfg.T, cfg.T // 16)) + [cfg.T - 1]
    olay = O.mx_blob_layout(cfg.H, cfg.I)
    x = hostgen.x(cfg, 0, 0)
    wr = hostgen.w_router(cfg, 0)
    lg = O.router_logits(O.bf16_bits_to_f64(x), wr)
    need = set(O.topk(lg[toks], cfg.k).reshape(-1).tolist()) | {cfg.E}
    blobs = {e: hostgen.expert_blob_mx(cfg, 0, e, olay) for e in need}
    stride = wl.layout.slot_stride
    for e in [cfg.E, min(need)]:
        assert np.array_equal(wl.pool[e * stride:e * stride + olay.blob_bytes].cpu().numpy(),
                              blobs[e][:olay.blob_bytes]), "device pool bytes, expert %d" % e
    say("[gpu]   %s: oracle on %d tokens" % (cfg.name, len(toks)))
    ora = O.moe_layer(x, lambda e: blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, hostgen.w_shared_gate(cfg, 0),
                      w_router=wr, tokens=toks, fmt="mx")
    kw = dict(drawn_logits=False, x64=O.bf16_bits_to_f64(x), w_router=wr)
    res, ties, worst = resolve_h_near_ties(buf, ora, cfg, lambda e: blobs[e], kw["x64"])
    say("[gpu]   h near ties adopted: %d (largest distance %.2f of its window)" % (ties, worst))
    say("[gpu]   end to end: %s" % end_to_end_y(buf, ora))
    stats = compare_layer(buf, res, cfg.T, cfg.k, cfg.E, **kw)
    say("[gpu]   %s ok: %s" % (cfg.name, stats))
    # quantised h of the sampled rows, bit for bit against the oracle's MXFP8 of the kernel's h
    inv = buf.inv_perm.cpu().numpy()
    rows = sorted({int(inv[t * cfg.k + j]) for t in toks for j in range(cfg.k)} | {cfg.T * cfg.k + t for t in toks})
    m = B.MxWorkspace(wl.dims)
    rt = torch.as_tensor(rows, device="cuda")
    h = bf16_to_f64(buf.h.index_select(0, rt))
    hc, hs, _ = O.mxfp8_quantize(h)
    gq = buf.mx_ws[m.off_hq:m.off_hq + (cfg.T * cfg.k + cfg.T) * cfg.I].view(-1, cfg.I).index_select(0, rt)
    gs = buf.mx_ws[m.off_hs:m.off_hs + (cfg.T * cfg.k + cfg.T) * m.hs_stride].view(-1, m.hs_stride)[:, :cfg.I // 32]
    gs = gs.index_select(0, rt)
    assert np.array_equal(gq.cpu().numpy(), hc) and np.array_equal(gs.cpu().numpy(), hs)
    # the step captured in a HIP graph: three replays, eager work between them,
    # each bit-identical to the eager run
    want = buf.y.view(torch.int16).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.run_step(0)
    for _ in range(3):
        buf.y.zero_()
        wl.run_step(0)
        torch.cuda.synchronize()
        buf.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.y.view(torch.int16), want), "graph replay differs from eager"
    del wl
    torch.cuda.empty_cache()


RGF_MX = {
    "decode48_window": Config(101, "rm1", T=4, H=2048, I=512, E=512, k=10, L=1, router="zipf", zipf_s=1.0, fmt="mx"),
    "t16_k6": Config(102, "rm2", T=16, H=512, I=256, E=256, k=6, L=1, router="zipf", zipf_s=1.2, fmt="mx"),
    "t13_k5": Config(103, "rm3", T=13, H=256, I=128, E=40, k=5, L=1, router="zipf", zipf_s=0.7, fmt="mx"),
    "router_matrix": Config(104, "rm4", T=8, H=512, I=256, E=32, k=4, L=1, router="matrix", fmt="mx"),
    "prefill_gemm": Config(105, "rm5", T=256, H=256, I=128, E=8, k=2, L=1, router="zipf", zipf_s=1.0, fmt="mx"),
}


@pytest.mark.parametrize("name", list(RGF_MX))
def test_route_group_ffn_mx_matches_separate_calls(B, hostgen, name):
    """moe_route_group_ffn_mx (route + group + MXFP8(x) in one launch for
    decode windows, separate kernels otherwise) gives every output of
    moe_route_group then moe_expert_ffn_mx bit for bit: ids, weights, sigma,
    offsets, perm, inv_perm, group_slot, status, the live rows of h and Y, and
    y after the combine; twice in a row, and with stages 1 then the down stage
    alone."""
    cfg = RGF_MX[name]
    say("[gpu] route + group + MX FFN %s (T=%d H=%d I=%d E=%d k=%d)" % (name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
    c = MxCase(B, cfg, hostgen)
    b = c.buf
    lg_in = None if c.wr_t is not None else c.logits_t
    lg_out = b.logits if c.wr_t is not None else None

    def call(mode):
        for t in (b.ids, b.offsets, b.perm, b.inv_perm, b.group_slot):
            t.fill_(-5)
        for t in (b.w, b.sigma):
            t.fill_(7.0)
        for t in (b.h, b.y_rows, b.y):
            t.fill_(3.0)
        b.status.zero_()
        b.mx_ws.fill_(0x5A)
        if mode == "separate":
            B.moe_route_group(c.dims, 0, c.x, c.wr_t, lg_in, c.wsg_t, lg_out, b.ids, b.w, b.sigma, c.slot_table,
                              cfg.E1, b.offsets, b.perm, b.inv_perm, b.group_slot, b.status, b.ws)
            B.moe_expert_ffn_mx(c.dims, c.x, c.pool, c.pool_bytes, c.layout, b.offsets, b.perm, b.group_slot, b.h,
                                b.y_rows, b.status, b.ws, b.mx_ws)
        else:
            B.moe_route_group_ffn_mx(c.dims, 0, c.x, c.wr_t, lg_in, c.wsg_t, lg_out, b.ids, b.w, b.sigma,
                                     c.slot_table, cfg.E1, b.offsets, b.perm, b.inv_perm, b.group_slot, c.pool,
                                     c.pool_bytes, c.layout, b.h, b.y_rows, b.status, b.ws, b.mx_ws,
                                     1 if mode == "fused_split" else 3)
            if mode == "fused_split":
                B.moe_expert_ffn_mx(c.dims, c.x, c.pool, c.pool_bytes, c.layout, b.offsets, b.perm, b.group_slot,
                                    b.h, b.y_rows, b.status, b.ws, b.mx_ws, 2)
        B.moe_combine(c.dims, b.y_rows, b.inv_perm, b.w, b.sigma, b.y)
        torch.cuda.synchronize()
        off = b.offsets.clone()
        live = torch.cat([torch.arange(int(off[cfg.E].item())),
                          torch.arange(cfg.T * cfg.k, cfg.T * cfg.k + cfg.T)]).cuda()
        return dict(ids=b.ids.clone(), w=b.w.view(torch.int32).clone(), sigma=b.sigma.view(torch.int32).clone(),
                    offsets=off, perm=b.perm.clone(), inv_perm=b.inv_perm.clone(),
                    group_slot=b.group_slot.clone(), status=b.status.clone(),
                    h=b.h.view(torch.int16)[live].clone(), y_rows=b.y_rows.view(torch.int16)[live].clone(),
                    y=b.y.view(torch.int16).clone())

    want = call("separate")
    assert int(want["status"].item()) == 0
    for mode in ("fused", "fused", "fused_split"):
        got = call(mode)
        for key in want:
            assert torch.equal(got[key], want[key]), "%s: %s differs" % (mode, key)

"""GPU parity of the MX variant: MXFP4 experts, MXFP8 activations, scaled MFMA.

- MXFP8 quantisation (moe_quantize_mxfp8): codes and scales bit for bit
  against the oracle, on values that span the E8M0 range, zero blocks, bf16
  subnormals, saturation and E4M3 ties.
- Whole layers through moe_expert_ffn_mx against oracle.moe_layer(fmt="mx"):
  ids, groups bit-exact; h, Y and y to the float bar of gpu_util against the
  oracle's own chain (no kernel value is fed to the oracle).  The workspace's
  quantised x and h are also checked bit for bit against the oracle's
  quantisation of the same bf16 values (x, and the kernel's own h), and, as a
  diagnostic, each stage against the oracle started from the kernel's output
  of the stage before (downstream_from_kernel_h).
- Where the scaled MFMA cannot meet the per-element bar: the instruction sums
  each 32-value block to about 13 bits below the block's largest product, so
  the kernel's h differs from the oracle's in the last bf16 bit on a few per
  cent of elements; MXFP8(h) then moves by a whole E4M3 step on some of them
  and those steps add up in Y and y.  The cases measured above the bar are
  marked xfail(strict=True) with their figure, so a change that fixes them
  shows up as an unexpected pass.
- Edge cases:
  - a one-step K (I = 128);
  - an odd step count (H = 384);
  - groups over two 256-row chunks and ragged tails;
  - a non-resident group;
  - stages split;
  - the device pool generator against the host one.
- Decode-sized groups (T k < 16 E): the weight-streaming kernel on MX blobs,
  its A rows the bf16 values of MXFP8(x) and MXFP8(h), both bit for bit
  against the oracle's quantisation; a K split into several rounds (H = 4608).
- Full size: prefill8192_mx on 17 sampled tokens."""
import numpy as np
import pytest
import torch

from gpu_util import compare_layer, say, bf16_to_f64
from oracle import moe_oracle as O
from synth import CONFIGS, Config, HostGen, DevGen, zipf_logits

pytestmark = pytest.mark.gpu


def downstream_from_kernel_h(buf, ora, cfg, blob_of):
    """A copy of the oracle's result in which each stage starts from the
    kernel's rounded output of the stage before: expert rows Y from the
    kernel's bf16 h (O.down_mx: the MXFP8 decision on h and the down
    projection), and y from the kernel's bf16 Y rows (O.combine).  Every
    rounding decision (R1, RA, R3) is then taken on the same values on both
    sides, and each stage is held to the float bar on its own.

    Why: the scaled MFMA sums each 32-value block to about 13 significant bits
    below the block's largest product (measured), about 1e-4 of an output,
    which flips the bf16 rounding of h and Y on a few per cent of elements.
    A flip of h can move its MXFP8 code by a step (or its block's shared
    exponent), and flipped Y units add up in y.  h itself is still compared
    with the oracle's own h, and y with the oracle's own y in relative L2."""
    import copy
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    olay = O.mx_blob_layout(H, I)
    new = copy.copy(ora)
    new.y_rows, new.y_rows_pre = dict(ora.y_rows), dict(ora.y_rows_pre)
    off = ora.groups.offsets
    by_e = {}
    for p in ora.y_rows:
        e = E if p >= T * k else int(np.searchsorted(off[:E + 1], p, side="right") - 1)
        by_e.setdefault(e, []).append(p)
    for e, rows in by_e.items():
        h = bf16_to_f64(buf.h.index_select(0, torch.as_tensor(rows, device=buf.h.device)))
        y_pre, y = O.down_mx(h, O.mx_dequant(blob_of(e), olay, 2, H, I))
        for i, p in enumerate(rows):
            new.y_rows_pre[p], new.y_rows[p] = y_pre[i], y[i]
    inv = ora.groups.inv_perm
    tok = [int(t) for t in ora.tokens]
    rows = [int(inv[t * k + j]) for t in tok for j in range(k)] + [T * k + t for t in tok]
    yk = bf16_to_f64(buf.y_rows.index_select(0, torch.as_tensor(rows, device=buf.y_rows.device)))
    n = len(tok)
    new.y_pre, new.y = O.combine(yk[:n * k].reshape(n, k, H), ora.w[tok], ora.sigma[tok], yk[n * k:])
    return new


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
        """The diagnostic (each stage from the kernel's previous stage), then
        the bar against the oracle's own chain."""
        kw = dict(drawn_logits=self.logits is not None, x64=O.bf16_bits_to_f64(self.x_bits), w_router=self.wr)
        staged = downstream_from_kernel_h(self.buf, ora, self.cfg, lambda e: self.blobs[e])
        diag = compare_layer(self.buf, staged, self.cfg.T, self.cfg.k, self.cfg.E, **kw)
        say("[gpu]   chained diagnostic: %s" % diag)
        say("[gpu]   end to end: %s" % end_to_end_y(self.buf, ora))
        return compare_layer(self.buf, ora, self.cfg.T, self.cfg.k, self.cfg.E, **kw)

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


# The scaled-MFMA cases measured above the per-element bar against the
# independent oracle (expert rows Y beyond 2e-2 rms + 2^-7 |ref|; y's largest
# element error as a multiple of rms(y)); strict, so a fix shows up as XPASS.
MX_BEYOND_BAR = {
    "mx_multichunk": "Y rows exceed the bound by 2.8e-4 (max |d| 9.8e-4, rms 3.3e-2); y max |d| 0.0221 rms",
    "mx_zipf": "Y rows exceed the bound by 3.8e-4 (max |d| 7.3e-4, rms 1.7e-2); y max |d| 0.0219 rms",
    "mx_many_items": "Y rows exceed the bound by 2.5e-3 (max |d| 3.9e-3, rms 4.7e-2); y max |d| 0.0353 rms",
}


@pytest.mark.parametrize("name", [pytest.param(n, marks=pytest.mark.xfail(
    strict=True, reason="scaled MFMA block-sum truncation moves MXFP8(h) codes: " + MX_BEYOND_BAR[n]))
    if n in MX_BEYOND_BAR else n for n in MX_SMALL])
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
    staged = downstream_from_kernel_h(buf, ora, cfg, lambda e: blobs[e])
    say("[gpu]   chained diagnostic: %s" % compare_layer(buf, staged, cfg.T, cfg.k, cfg.E, drawn_logits=True))
    say("[gpu]   end to end: %s" % end_to_end_y(buf, ora))
    stats = compare_layer(buf, ora, cfg.T, cfg.k, cfg.E, drawn_logits=True)
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
    staged = downstream_from_kernel_h(buf, ora, cfg, lambda e: blobs[e])
    kw = dict(drawn_logits=False, x64=O.bf16_bits_to_f64(x), w_router=wr)
    say("[gpu]   chained diagnostic: %s" % compare_layer(buf, staged, cfg.T, cfg.k, cfg.E, **kw))
    say("[gpu]   end to end: %s" % end_to_end_y(buf, ora))
    stats = compare_layer(buf, ora, cfg.T, cfg.k, cfg.E, **kw)
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

"""GPU tests of the measurement probes: the read probe reads and writes nothing
for ordinary data; the bf16 MFMA probe's sums equal what the MFMAs it issues
must produce (exact: every value is a small multiple of 2^-7); the scaled
fp8/fp4 MFMA probes give the same finite result in every workgroup."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


def test_read_probe_reads_without_writing(B):
    buf = torch.full((64 << 20,), 1, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    B.moe_probe_hbm_read(buf, buf.numel(), 512, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def _bf16_probe_wave_sum(iters):
    """Sum over one wavefront's 64 lanes of the probe's kind-0 output: 4
    accumulators x iters x sum_ij (A B)[i][j], where lane l holds
    A[l % 32][8 (l // 32) + e] = ((l + e) & 7) / 8 and
    B[8 (l // 32) + e][l % 32] = ((3 l + e) & 7) / 16; the sum over all of D
    is sum_k colsum_A[k] rowsum_B[k]."""
    tot = 0.0
    for q in range(2):
        lanes = range(32 * q, 32 * q + 32)
        for e in range(8):
            ca = sum(((l + e) & 7) / 8.0 for l in lanes)
            rb = sum(((3 * l + e) & 7) / 16.0 for l in lanes)
            tot += ca * rb
    return 4 * iters * tot


def test_mfma_probes(B):
    grid, iters = 8, 64
    for kind in (0, 1, 2):
        sink = torch.zeros(grid * 256, dtype=torch.float32, device="cuda")
        B.moe_probe_mfma(kind, grid, iters, sink)
        torch.cuda.synchronize()
        v = sink.cpu().numpy().astype(np.float64).reshape(grid, 4, 64)
        say("[gpu] mfma probe kind %d: lane sums %s" % (kind, v[0, 0, :4]))
        assert np.isfinite(v).all() and np.abs(v).sum() > 0
        assert (v == v[:1, :1]).all(), "every wavefront issues the same MFMAs"
        if kind == 0:
            assert v[0, 0].sum() == _bf16_probe_wave_sum(iters)


# ---- the scaled MFMA's arithmetic and the gate/up split ------------------------

def _pack_scaled(A, B, SA, SB):
    """Logical operands -> the instruction's lanes (moe_probe_scaled_mfma).
    A uint8 E4M3 codes [n, 16, 128]; B E2M1 nibbles [n, 128, 16]; SA, SB E8M0
    bytes [n, 16, 4] (row / column, K block)."""
    n = A.shape[0]
    pa = np.zeros((n, 64, 8), np.uint32)
    pb = np.zeros((n, 64, 4), np.uint32)
    psa = np.zeros((n, 64), np.int32)
    psb = np.zeros((n, 64), np.int32)
    for l in range(64):
        i, j = l % 16, l // 16
        ks = list(range(16 * j, 16 * j + 16)) + list(range(64 + 16 * j, 64 + 16 * j + 16))
        by = A[:, i, ks].astype(np.uint32)
        pa[:, l] = by[:, 0::4] | (by[:, 1::4] << 8) | (by[:, 2::4] << 16) | (by[:, 3::4] << 24)
        nib = B[:, 32 * j:32 * j + 32, i].astype(np.uint32)
        byt = nib[:, 0::2] | (nib[:, 1::2] << 4)
        pb[:, l] = byt[:, 0::4] | (byt[:, 1::4] << 8) | (byt[:, 2::4] << 16) | (byt[:, 3::4] << 24)
        psa[:, l] = SA[:, i, j]
        psb[:, l] = SB[:, i, j]
    return [torch.from_numpy(np.ascontiguousarray(v).view(np.int32)).cuda() for v in (pa, pb, psa, psb)]


def _run_scaled(B, A, Bc, SA, SB, split):
    n = A.shape[0]
    pa, pb, psa, psb = _pack_scaled(A, Bc, SA, SB)
    d = torch.zeros((n, 64, 4), dtype=torch.float32, device="cuda")
    B.moe_probe_scaled_mfma(pa, pb, psa, psb, n, split, d)
    torch.cuda.synchronize()
    d = d.cpu().numpy().astype(np.float64)
    out = np.zeros((n, 16, 16))
    for l in range(64):
        for e in range(4):
            out[:, 4 * (l // 16) + e, l % 16] = d[:, l, e]
    return out


def _exact_scaled(A, Bc, SA, SB):
    """sum_k a b exactly (fp64 holds every product and block sum), and sum_k |a b|."""
    from oracle import moe_oracle as O
    a = O.e4m3fn_decode(A)
    b = O.e2m1_decode(Bc)
    sa, sb = O.e8m0_decode(SA), O.e8m0_decode(SB)
    ex = np.zeros((A.shape[0], 16, 16))
    ab = np.zeros_like(ex)
    for j in range(4):
        k = slice(32 * j, 32 * j + 32)
        sc = sa[:, :, j][:, :, None] * sb[:, :, j][:, None, :]
        ex += np.matmul(a[:, :, k], b[:, k, :]) * sc
        ab += np.matmul(np.abs(a[:, :, k]), np.abs(b[:, k, :])) * sc
    return ex, ab


def test_scaled_mfma_truncates_inside_a_run_and_the_split_does_not(B):
    """One run of 8 products holding 256 x 1 and a small code x 1 (every E4M3
    code below 2, subnormals included): the instruction keeps the small product
    only down to 2^(8 - 13), truncated toward zero; the split pair sums it whole."""
    from oracle import moe_oracle as O
    codes = np.array([c for c in range(1, 0x40)] + [0x80 | c for c in range(1, 0x40)], np.uint8)
    n = codes.size
    A = np.zeros((n, 16, 128), np.uint8)
    Bc = np.zeros((n, 128, 16), np.uint8)
    A[:, 0, 0] = 0x78           # 256
    A[:, 0, 1] = codes
    Bc[:, 0, 0] = Bc[:, 1, 0] = 0x2   # 1.0
    S = np.full((n, 16, 4), 127, np.uint8)
    small = O.e4m3fn_decode(codes)
    want_hw = 256.0 + np.trunc(small / 2.0 ** -5) * 2.0 ** -5
    got = _run_scaled(B, A, Bc, S, S, 0)[:, 0, 0]
    assert np.array_equal(got, want_hw), "run truncation below 2^(m - 13)"
    assert np.count_nonzero(got != 256.0 + small) > 0
    got2 = _run_scaled(B, A, Bc, S, S, 1)[:, 0, 0]
    assert np.array_equal(got2, 256.0 + small), "the split sums every product whole"


@pytest.mark.parametrize("kind", ["x", "h"])
def test_split_sums_mxfp8_blocks_whole(B, kind):
    """MXFP8 rows as the GEMM sees them (x: N(0, 1); h: silu(g) u of two N(0, 1))
    against random E2M1 columns and E8M0 scales: the split pair is the exact
    sum up to fp32 addition (<= 2^-21 of sum |products|), the single MFMA is not."""
    from oracle import moe_oracle as O
    rng = np.random.default_rng(17 if kind == "x" else 18)
    n = 96
    if kind == "x":
        v = rng.standard_normal((n * 16, 128))
    else:
        g, u = rng.standard_normal((2, n * 16, 128))
        v = g / (1.0 + np.exp(-g)) * u
    codes, scales, _ = O.mxfp8_quantize(v)
    A = codes.reshape(n, 16, 128)
    SA = scales.reshape(n, 16, 4)
    Bc = rng.integers(0, 16, size=(n, 128, 16)).astype(np.uint8)
    SB = rng.integers(118, 125, size=(n, 16, 4)).astype(np.uint8)
    ex, ab = _exact_scaled(A, Bc, SA, SB)
    split = np.abs(_run_scaled(B, A, Bc, SA, SB, 1) - ex) / ab
    single = np.abs(_run_scaled(B, A, Bc, SA, SB, 0) - ex) / ab
    say("[gpu] scaled MFMA on %s-like MXFP8 rows: |err| / sum|p| split %.3g, single %.3g" % (
        kind, split.max(), single.max()))
    assert split.max() <= 2.0 ** -21
    assert single.max() > 2.0 ** -18

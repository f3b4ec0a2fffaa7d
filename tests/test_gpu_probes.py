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

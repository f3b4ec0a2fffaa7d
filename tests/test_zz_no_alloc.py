"""The entry point that allocates nothing, moe_expert_ffn_mx_noalloc, against
moe_expert_ffn_mx with a caller workspace: h and the expert rows Y bit for bit,
on two calls in a row (the second on a smaller input, so it reuses the
library's static scratch after a larger call left other contents there), on
both FFN paths (grouped GEMM on the scaled MFMA, then weight streaming)."""
import pytest
import torch

from gpu_util import say
from synth import Config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


# the larger call first: groups over two 256-row chunks (grouped GEMM); then a
# decode window (weight streaming), whose workspace is a different layout
CASES = [
    Config(52, "mxm", T=700, H=512, I=256, E=4, k=2, L=1, router="matrix", fmt="mx"),
    Config(61, "mxd", T=4, H=256, I=128, E=32, k=4, L=1, router="zipf", zipf_s=1.0, fmt="mx"),
]


def test_noalloc_matches_caller_workspace_on_two_calls(B, hostgen):
    from test_gpu_mx import MxCase
    need = [B.moe_mx_workspace_bytes(B.Dims(c.T, c.H, c.I, c.E, c.k, 1)) for c in CASES]
    assert need[1] < need[0] <= 32 << 20
    for cfg in CASES:
        say("[gpu] no-alloc FFN vs caller workspace (T=%d H=%d I=%d E=%d k=%d)" % (cfg.T, cfg.H, cfg.I, cfg.E, cfg.k))
        c = MxCase(B, cfg, hostgen)
        c.run(B)   # route, group, FFN with the caller's MX workspace, combine
        assert int(c.buf.status.item()) == 0
        want_h = c.buf.h.view(torch.int16).clone()
        want_y = c.buf.y_rows.view(torch.int16).clone()
        buf = c.buf
        buf.h.fill_(1.0)
        buf.y_rows.fill_(1.0)
        B.moe_expert_ffn_mx_noalloc(c.dims, c.x, c.pool, c.pool_bytes, c.layout, buf.offsets, buf.perm,
                                    buf.group_slot, buf.h, buf.y_rows, buf.status, buf.ws)
        torch.cuda.synchronize()
        assert int(buf.status.item()) == 0
        # rows of groups that exist (rows past offsets[E] belong to dropped ids and are not written)
        nr = cfg.T * cfg.k + cfg.T
        off_e = int(buf.offsets[cfg.E].item())
        live = torch.cat([torch.arange(off_e), torch.arange(cfg.T * cfg.k, nr)]).cuda()
        assert torch.equal(buf.h.view(torch.int16)[live], want_h[live]), "h differs"
        assert torch.equal(buf.y_rows.view(torch.int16)[live], want_y[live]), "Y rows differ"
        # the stages apart: gate/up, then down, through the same scratch
        buf.h.fill_(1.0)
        buf.y_rows.fill_(1.0)
        for st in (1, 2):
            B.moe_expert_ffn_mx_noalloc(c.dims, c.x, c.pool, c.pool_bytes, c.layout, buf.offsets, buf.perm,
                                        buf.group_slot, buf.h, buf.y_rows, buf.status, buf.ws, stages=st)
        torch.cuda.synchronize()
        assert torch.equal(buf.y_rows.view(torch.int16)[live], want_y[live]), "Y rows differ (stages apart)"
        del c
        torch.cuda.empty_cache()

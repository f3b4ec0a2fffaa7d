"""GPU tests of partial residency (the LRU cache of expert blobs).

The residency kernel is compared with the oracle's LRU cache step by step on
random traces (slot table, owners, last uses, clock, fill list and count, bit
for bit), including a cache of 3000 slots where many slots share a last use,
and the overflow case.  A whole decode run through a cache smaller than the
experts it touches, filled from pinned host memory by the fixed-shape fill
kernel, gives the all-resident run's outputs bit for bit ([FreeToken] 3.3 and 4:
the cache changes where blobs live, never what is computed)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import say
from oracle import moe_oracle as O
from synth import Config, HostGen, zipf_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


class DevCache:
    """The cache state on the device, initialised empty."""

    def __init__(self, L, E, S):
        i32 = dict(dtype=torch.int32, device="cuda")
        self.slot_table = torch.full((L, E + 1), -1, **i32)
        self.owner = torch.full((S,), -1, **i32)
        self.last = torch.full((S,), -1, **i32)
        self.clock = torch.zeros(1, **i32)
        self.fills = torch.full((E + 1, 2), -7, **i32)
        self.n_fill = torch.zeros(1, **i32)
        self.status = torch.zeros(1, **i32)
        self.S = S

    def update(self, B, dims, layer, ids):
        B.moe_residency_update(dims, layer, ids, self.slot_table, self.owner, self.last, self.S, self.clock,
                               self.fills, self.n_fill, self.status)


@pytest.mark.parametrize("L,E,S,T,k", [(3, 8, 10, 2, 3), (2, 64, 100, 4, 8), (4, 512, 3000, 4, 10)])
def test_residency_matches_lru_oracle(B, L, E, S, T, k):
    say("[gpu] residency trace L=%d E=%d S=%d T=%d k=%d" % (L, E, S, T, k))
    rng = np.random.default_rng(L * 1000 + E + S)
    dims = B.Dims(T, 64, 32, E, k, L)
    dev, ora = DevCache(L, E, S), O.LruCache(L, E, S)
    ids_t = torch.empty((T, k), dtype=torch.int32, device="cuda")
    hot = rng.choice(E, size=min(E, 3 * k), replace=False)   # a hot set, so hits happen
    for i in range(60):
        layer = i % L
        ids = np.stack([rng.choice(hot if rng.random() < 0.7 else np.arange(E), size=k, replace=False)
                        for _ in range(T)]).astype(np.int32)
        ids_t.copy_(torch.from_numpy(ids))
        dev.update(B, dims, layer, ids_t)
        fills, full = ora.step(layer, ids)
        torch.cuda.synchronize()
        n = int(dev.n_fill.item())
        assert n == len(fills) and not full and int(dev.status.item()) == 0, "call %d" % i
        assert [tuple(r) for r in dev.fills[:n].cpu().numpy()] == fills, "call %d" % i
        assert np.array_equal(dev.slot_table.cpu().numpy(), ora.slot_table), "call %d" % i
        assert np.array_equal(dev.owner.cpu().numpy(), ora.owner), "call %d" % i
        assert np.array_equal(dev.last.cpu().numpy(), ora.last), "call %d" % i
        assert int(dev.clock.item()) == ora.clock


def test_residency_overflow_sets_status(B):
    say("[gpu] residency overflow")
    L, E, S, T, k = 1, 6, 3, 2, 2
    dims = B.Dims(T, 64, 32, E, k, L)
    dev, ora = DevCache(L, E, S), O.LruCache(L, E, S)
    ids = np.array([[0, 1], [2, 3]], np.int32)   # four routed + the shared expert: 5 > 3 slots
    dev.update(B, dims, 0, torch.from_numpy(ids).cuda())
    fills, full = ora.step(0, ids)
    torch.cuda.synchronize()
    assert full and int(dev.status.item()) == B.MOE_DEV_CACHE_FULL
    assert int(dev.n_fill.item()) == 3 and [tuple(r) for r in dev.fills[:3].cpu().numpy()] == fills
    assert np.array_equal(dev.slot_table.cpu().numpy(), ora.slot_table)


def _device_pointer(host_ptr):
    """The device-readable address of pinned host memory (None if HIP has none)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    out = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(host_ptr), 0)
    return out.value if rc == 0 and out.value else None


def test_decode_through_a_small_cache_matches_all_resident(B, hostgen):
    """Two layers, windows of 4 tokens over 6 steps; the cache holds 24 of the
    34 blobs, so layers evict each other's experts.  Every step's output is the
    all-resident output, bit for bit, and every cached slot holds its key's bytes."""
    from moe_expert_ffn_top_amd.layer import LayerBuffers
    cfg = Config(43, "pr", T=4, H=128, I=64, E=16, k=4, L=2, router="zipf", zipf_s=0.8)
    L, E, T, k = cfg.L, cfg.E, cfg.T, cfg.k
    E1, S = E + 1, 24
    say("[gpu] decode through a %d-slot cache (L=%d, E=%d)" % (S, L, E))
    lay = B.moe_blob_layout_init(cfg.H, cfg.I)
    olay = O.blob_layout(cfg.H, cfg.I)
    stride = lay.slot_stride
    blobs = np.zeros((L * E1, stride), np.uint8)
    for l in range(L):
        for e in range(E1):
            b = hostgen.expert_blob(cfg, l, e, olay)
            blobs[l * E1 + e, :len(b)] = b
    host = torch.empty(blobs.size, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = blobs.reshape(-1)
    dptr = _device_pointer(host.data_ptr())
    if dptr is None:
        pytest.skip("pinned host memory has no device address here")
    full_pool = torch.from_numpy(blobs.reshape(-1).copy()).cuda()
    full_table = torch.arange(L * E1, dtype=torch.int32, device="cuda").view(L, E1).contiguous()
    pool = torch.zeros(S * stride, dtype=torch.uint8, device="cuda")
    dims = B.Dims(T, cfg.H, cfg.I, E, k, L)
    dev = DevCache(L, E, S)
    wsg = torch.from_numpy(hostgen.w_shared_gate(cfg, 0)).cuda()
    a, b = LayerBuffers.allocate(dims), LayerBuffers.allocate(dims)
    for step in range(6):
        for l in range(L):
            x = torch.from_numpy(hostgen.x(cfg, l, step).view(np.int16)).cuda().view(torch.bfloat16)
            lg = torch.from_numpy(zipf_logits(cfg, l, step)).cuda()
            for buf, table, p, n_slots in ((a, full_table, full_pool, L * E1), (b, None, pool, S)):
                B.moe_route(dims, x, None, lg, wsg, None, buf.ids, buf.w, buf.sigma)
                if table is None:
                    dev.update(B, dims, l, buf.ids)
                    B.moe_residency_fill(dims, lay, dptr, pool, pool.numel(), S, dev.fills, dev.n_fill)
                    table = dev.slot_table
                buf.status.zero_()
                B.moe_group(dims, l, buf.ids, table, n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                            buf.status, buf.ws)
                B.moe_expert_ffn(dims, x, p, p.numel(), lay, buf.offsets, buf.perm, buf.group_slot, buf.h,
                                 buf.y_rows, buf.status, buf.ws)
                B.moe_combine(dims, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y)
            torch.cuda.synchronize()
            assert int(b.status.item()) == 0 and int(dev.status.item()) == 0, "step %d layer %d" % (step, l)
            assert torch.equal(a.ids, b.ids)
            assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16)), "step %d layer %d" % (step, l)
    owner = dev.owner.cpu().numpy()
    cached = pool.view(S, stride).cpu().numpy()
    for s in range(S):
        if owner[s] >= 0:
            assert np.array_equal(cached[s, :lay.blob_bytes], blobs[owner[s], :lay.blob_bytes]), "slot %d" % s
    assert int(dev.clock.item()) == 6 * L

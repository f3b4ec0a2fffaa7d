"""GPU tests of the hot/cold swap policy's device side.

Heat accumulated from moe_group's offsets and decayed on the device equals the
oracle's fp32 heat bit for bit over a random routing sequence; moe_swap_apply
moves each planned hot expert's blob into its cold partner's slot, publishes
the table, leaves every other slot alone and skips a plan entry that no longer
fits the table ([Strata] "哪些专家能长期留在显存？")."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import say
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


def test_heat_matches_oracle(B):
    from moe_expert_ffn_top_amd.layer import LayerBuffers
    L, E, T, k = 3, 40, 6, 4
    say("[gpu] heat accumulation L=%d E=%d" % (L, E))
    d = B.Dims(T, 64, 32, E, k, L)
    buf = LayerBuffers.allocate(d)
    st = torch.arange(L * (E + 1), dtype=torch.int32, device="cuda").view(L, E + 1).contiguous()
    heat = torch.zeros((L, E), dtype=torch.float32, device="cuda")
    ref = np.zeros((L, E), np.float32)
    rng = np.random.default_rng(11)
    for i in range(30):
        layer = i % L
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        buf.ids.copy_(torch.from_numpy(ids))
        B.moe_group(d, layer, buf.ids, st, L * (E + 1), buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                    buf.status, buf.ws)
        B.moe_heat_update(d, layer, buf.offsets, heat)
        O.heat_add(ref, layer, ids)
        if i % 7 == 6:
            B.moe_heat_decay(d, heat, 0.7)
            O.heat_decay(ref, 0.7)
    torch.cuda.synchronize()
    assert np.array_equal(heat.cpu().numpy(), ref)


def _device_pointer(host_ptr):
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    out = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(host_ptr), 0)
    return out.value if rc == 0 and out.value else None


def test_swap_apply_moves_blobs_and_publishes(B):
    L, E, H, I = 2, 8, 64, 32
    E1 = E + 1
    say("[gpu] swap apply L=%d E=%d" % (L, E))
    lay = B.moe_blob_layout_init(H, I)
    stride = lay.slot_stride
    rng = np.random.default_rng(4)
    blobs = rng.integers(0, 256, size=(L * E1, stride), dtype=np.uint8)
    host = torch.empty(blobs.size, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = blobs.reshape(-1)
    dptr = _device_pointer(host.data_ptr())
    if dptr is None:
        pytest.skip("pinned host memory has no device address here")
    # residents: experts 4..7 and the shared one of each layer, in slots 0..9
    table = np.full((L, E1), -1, np.int32)
    n = 0
    for l in range(L):
        for e in list(range(4, E)) + [E]:
            table[l, e] = n
            n += 1
    S = n
    pool_np = np.zeros((S, stride), np.uint8)
    for l in range(L):
        for e in range(E1):
            if table[l, e] >= 0:
                pool_np[table[l, e]] = blobs[l * E1 + e]
    pool = torch.from_numpy(pool_np.reshape(-1).copy()).cuda()
    heat = np.zeros((L, E), np.float32)
    heat[0, :4] = [9, 2, 7, 0]
    heat[0, 4:] = [1, 6, 0, 5]
    heat[1, :4] = [3, 3, 3, 3]
    heat[1, 4:] = [3, 3, 3, 0]
    d = B.Dims(1, H, I, E, 1, L)
    plan = B.moe_swap_plan(d, heat, table)
    want = O.swap_plan(heat, table)
    assert [tuple(r) for r in plan] == want and len(want) == 3
    plan_dev = np.concatenate([plan, [[0, 5, 6]]]).astype(np.int32)   # a stale entry: expert 5 stays resident
    t_dev = torch.from_numpy(table.copy()).cuda()
    scratch = torch.zeros((len(plan_dev), 2), dtype=torch.int32, device="cuda")
    nsc = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_swap_apply(d, lay, dptr, pool, pool.numel(), S, t_dev, torch.from_numpy(plan_dev).cuda(), len(plan_dev),
                     scratch, nsc)
    torch.cuda.synchronize()
    exp_table, exp_pool = table.copy(), pool_np.copy()
    for l, hot, cold in want:
        s = table[l, cold]
        exp_table[l, hot], exp_table[l, cold] = s, -1
        exp_pool[s, :lay.blob_bytes] = blobs[l * E1 + hot, :lay.blob_bytes]
    assert np.array_equal(t_dev.cpu().numpy(), exp_table)
    assert np.array_equal(pool.view(S, stride).cpu().numpy(), exp_pool)


def test_swap_apply_skips_entries_naming_an_expert_twice(B):
    """A plan that names one expert in two entries of a layer (as hot or as
    cold) applies only the first of them: two fills into one slot, or one
    expert moved twice, would leave the table naming bytes of another expert."""
    L, E, H, I = 1, 8, 64, 32
    E1 = E + 1
    say("[gpu] swap apply: repeated experts in a plan")
    lay = B.moe_blob_layout_init(H, I)
    stride = lay.slot_stride
    rng = np.random.default_rng(9)
    blobs = rng.integers(0, 256, size=(L * E1, stride), dtype=np.uint8)
    host = torch.empty(blobs.size, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = blobs.reshape(-1)
    dptr = _device_pointer(host.data_ptr())
    if dptr is None:
        pytest.skip("pinned host memory has no device address here")
    table = np.full((L, E1), -1, np.int32)
    for s, e in enumerate(list(range(4, E)) + [E]):   # experts 4..7 and the shared one resident
        table[0, e] = s
    S = 5
    pool_np = np.zeros((S, stride), np.uint8)
    for e in range(E1):
        if table[0, e] >= 0:
            pool_np[table[0, e]] = blobs[e]
    pool = torch.from_numpy(pool_np.reshape(-1).copy()).cuda()
    d = B.Dims(1, H, I, E, 1, L)
    # an entry is checked against every earlier entry, applied or skipped
    plan = np.array([[0, 0, 6],    # applied
                     [0, 1, 6],    # cold 6 again: skipped
                     [0, 0, 4],    # hot 0 again: skipped
                     [0, 2, 4],    # cold 4 named by the (skipped) entry before: skipped
                     [0, 3, 7],    # applied (experts named by no earlier entry)
                     [0, 6, 5]],   # names 6, already a cold of entry 0: skipped
                    np.int32)
    t_dev = torch.from_numpy(table.copy()).cuda()
    scratch = torch.zeros((len(plan), 2), dtype=torch.int32, device="cuda")
    nsc = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_swap_apply(d, lay, dptr, pool, pool.numel(), S, t_dev, torch.from_numpy(plan).cuda(), len(plan),
                     scratch, nsc)
    torch.cuda.synchronize()
    exp_table, exp_pool = table.copy(), pool_np.copy()
    for hot, cold in ((0, 6), (3, 7)):
        s = table[0, cold]
        exp_table[0, hot], exp_table[0, cold] = s, -1
        exp_pool[s, :lay.blob_bytes] = blobs[hot, :lay.blob_bytes]
    assert np.array_equal(t_dev.cpu().numpy(), exp_table)
    assert np.array_equal(pool.view(S, stride).cpu().numpy(), exp_pool)
    assert np.array_equal(scratch.cpu().numpy()[[1, 2, 3, 5], 0], [-1, -1, -1, -1])

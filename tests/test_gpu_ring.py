"""GPU tests of the two-slot staging ring's protocol ([Strata] "PCIe 搬运怎样与
计算重叠？": the compute stream waits for a slot's copy before reading it, and
the next copy into a slot waits until the compute stream is done with it).

- protocol misuse returns MOE_ERR_STATE and leaves the ring usable: staging
  into a slot that was not released, releasing before acquiring, acquiring
  twice, releasing twice, acquiring an empty slot;
- a pageable or device source returns MOE_ERR_NOT_PINNED, an oversized one
  MOE_ERR_ARG;
- delay injection with the protocol intact: a bounded busy kernel runs on the
  compute stream between a slot's acquire and the read that checks it, and
  the next layer is staged into that slot meanwhile.  The read sees the slot's
  own layer, never the next one: the copy waited for the release."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu

SLOT = 64 << 20


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_expert_ffn_top_amd import binding
    return binding


def _host_layers(n, seed):
    """n pinned host buffers of SLOT bytes with distinct seeded contents, and
    each one's checksum (int64 sum of its int32 words)."""
    rng = np.random.default_rng(seed)
    bufs, sums = [], []
    for _ in range(n):
        a = rng.integers(-2 ** 31, 2 ** 31, size=SLOT // 4, dtype=np.int64).astype(np.int32)
        t = torch.empty(SLOT, dtype=torch.uint8, pin_memory=True)
        t.view(torch.int32).copy_(torch.from_numpy(a))
        bufs.append(t)
        sums.append(int(a.astype(np.int64).sum()))
    return bufs, sums


def _checksum(slot):
    return slot.view(torch.int32).sum(dtype=torch.int64)


class _Ring:
    def __init__(self, B):
        self.B = B
        self.slots = [torch.zeros(SLOT, dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.copy = torch.cuda.Stream()
        self.comp = torch.cuda.Stream()
        self.r = B.moe_ring_create(self.slots[0], self.slots[1], SLOT, self.copy)

    def close(self):
        torch.cuda.synchronize()
        self.B.moe_ring_destroy(self.r)


def _status(B, fn):
    with pytest.raises(B.MoeError) as e:
        fn()
    return e.value.status


def test_ring_protocol_misuse_is_refused(B):
    say("[gpu] ring: protocol misuse")
    host, sums = _host_layers(3, 1)
    R = _Ring(B)
    try:
        assert B.moe_stage_h2d(R.r, host[0].data_ptr(), SLOT) == 0
        assert B.moe_stage_h2d(R.r, host[1].data_ptr(), SLOT) == 1
        # slot 0 holds layer 0, not yet released
        assert _status(B, lambda: B.moe_stage_h2d(R.r, host[2].data_ptr(), SLOT)) == B.MOE_ERR_STATE
        assert _status(B, lambda: B.moe_ring_release(R.r, 0, R.comp)) == B.MOE_ERR_STATE   # before acquire
        B.moe_ring_acquire(R.r, 0, R.comp)
        assert _status(B, lambda: B.moe_ring_acquire(R.r, 0, R.comp)) == B.MOE_ERR_STATE   # twice
        with torch.cuda.stream(R.comp):
            c0 = _checksum(R.slots[0])
        B.moe_ring_release(R.r, 0, R.comp)
        assert _status(B, lambda: B.moe_ring_release(R.r, 0, R.comp)) == B.MOE_ERR_STATE   # twice
        assert _status(B, lambda: B.moe_ring_acquire(R.r, 0, R.comp)) == B.MOE_ERR_STATE   # empty
        # the refused calls changed nothing: the next stage goes to slot 0
        assert B.moe_stage_h2d(R.r, host[2].data_ptr(), SLOT) == 0
        for s in (1, 0):
            B.moe_ring_acquire(R.r, s, R.comp)
            with torch.cuda.stream(R.comp):
                c = _checksum(R.slots[s])
            B.moe_ring_release(R.r, s, R.comp)
            if s == 1:
                c1 = c
            else:
                c2 = c
        torch.cuda.synchronize()
        assert [int(c0), int(c1), int(c2)] == sums
    finally:
        R.close()


def test_ring_refuses_unpinned_and_oversized_sources(B):
    say("[gpu] ring: pageable, device and oversized sources")
    R = _Ring(B)
    try:
        pageable = np.ones(SLOT, dtype=np.uint8)
        assert _status(B, lambda: B.moe_stage_h2d(R.r, pageable.ctypes.data, SLOT)) == B.MOE_ERR_NOT_PINNED
        dev = torch.ones(SLOT, dtype=torch.uint8, device="cuda")
        assert _status(B, lambda: B.moe_stage_h2d(R.r, dev.data_ptr(), SLOT)) == B.MOE_ERR_NOT_PINNED
        big = torch.ones(SLOT + 4096, dtype=torch.uint8, pin_memory=True)
        assert _status(B, lambda: B.moe_stage_h2d(R.r, big.data_ptr(), SLOT + 4096)) == B.MOE_ERR_ARG
        # nothing was staged, and the ring still works
        assert B.moe_stage_h2d(R.r, big.data_ptr(), SLOT) == 0
        B.moe_ring_acquire(R.r, 0, R.comp)
        with torch.cuda.stream(R.comp):
            c = _checksum(R.slots[0])
        B.moe_ring_release(R.r, 0, R.comp)
        torch.cuda.synchronize()
        assert int(c) == SLOT // 4 * 0x01010101
    finally:
        R.close()


def _sleep_cycles_for(ms):
    """Cycles of torch's bounded spin kernel that take about `ms` here."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 22
    torch.cuda._sleep(n)   # the first launch also loads the kernel
    a.record()
    torch.cuda._sleep(n)
    b.record()
    torch.cuda.synchronize()
    per_ms = n / max(1e-3, a.elapsed_time(b))
    return int(min(per_ms * ms, 4e9))


def test_ring_used_wait_holds_the_next_copy(B):
    """Layer 2 is staged into slot 0 while the compute stream is still busy
    before its read of layer 0 there; the read must still see layer 0."""
    say("[gpu] ring: delay injection before the release")
    host, sums = _host_layers(3, 2)
    cycles = _sleep_cycles_for(40.0)
    R = _Ring(B)
    try:
        assert B.moe_stage_h2d(R.r, host[0].data_ptr(), SLOT) == 0
        assert B.moe_stage_h2d(R.r, host[1].data_ptr(), SLOT) == 1
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        B.moe_ring_acquire(R.r, 0, R.comp)
        with torch.cuda.stream(R.comp):
            t0.record()
            torch.cuda._sleep(cycles)   # bounded busy kernel between acquire and the read
            c0 = _checksum(R.slots[0])
            t1.record()
        B.moe_ring_release(R.r, 0, R.comp)
        # enqueued while the spin still runs; a 64 MiB copy takes a few ms, so
        # without the wait on the release it would land inside the spin
        assert B.moe_stage_h2d(R.r, host[2].data_ptr(), SLOT) == 0
        done = []
        for s in (1, 0):
            B.moe_ring_acquire(R.r, s, R.comp)
            with torch.cuda.stream(R.comp):
                done.append(_checksum(R.slots[s]))
            B.moe_ring_release(R.r, s, R.comp)
        torch.cuda.synchronize()
        say("[gpu]   busy kernel + read of slot 0: %.1f ms" % t0.elapsed_time(t1))
        assert [int(c0), int(done[0]), int(done[1])] == sums
        # the spin outlasted a 64 MiB copy (a few ms at PCIe rates) many times over
        assert t0.elapsed_time(t1) > 5.0
    finally:
        R.close()

"""libmoe's C ABI on the CPU: it loads, exports what include/moe.h declares, its
host-pure functions agree with the format spec, and argument validation
returns the documented codes without enqueueing anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from oracle import moe_oracle as O


@pytest.fixture(scope="module")
def B():
    from moe_expert_ffn_top_amd import binding
    return binding


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(B):
    declared = _declared_functions()
    assert len(declared) >= 15
    assert sorted(B.EXPORTED) == declared
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(B):
    assert "gfx950" in B.moe_version()
    assert B.moe_status_string(0) == "MOE_OK"
    for code in range(-7, 0):
        assert B.moe_status_string(code).startswith("MOE_ERR_")


@pytest.mark.parametrize("H,I", [(32, 32), (512, 256), (2048, 512), (4096, 2048), (96, 160), (16384, 32)])
def test_blob_layout_matches_format_spec(B, H, I):
    lay = B.moe_blob_layout_init(H, I)
    ref = O.blob_layout(H, I)
    assert tuple(lay.off_codes) == ref.off_codes
    assert tuple(lay.off_scales) == ref.off_scales
    assert lay.off_globals == ref.off_globals
    assert lay.blob_bytes == ref.blob_bytes and lay.slot_stride == ref.slot_stride


@pytest.mark.parametrize("H,I", [(0, 32), (48, 32), (32, 16400), (32, -32)])
def test_blob_layout_rejects_bad_widths(B, H, I):
    with pytest.raises(B.MoeError) as e:
        B.moe_blob_layout_init(H, I)
    assert e.value.status == B.MOE_ERR_SHAPE


@pytest.mark.parametrize("dims,code", [
    ((0, 512, 256, 32, 4, 1), "MOE_ERR_SHAPE"),      # empty input: T = 0
    ((8, 500, 256, 32, 4, 1), "MOE_ERR_SHAPE"),      # H % 32 != 0
    ((8, 512, 256, 32, 33, 1), "MOE_ERR_SHAPE"),     # k > E
    ((8, 512, 256, 1025, 4, 1), "MOE_ERR_SHAPE"),    # E > 1024
    ((8, 512, 256, 32, 0, 1), "MOE_ERR_SHAPE"),      # k = 0
    ((8, 512, 256, 32, 4, 0), "MOE_ERR_SHAPE"),      # L = 0
])
def test_workspace_rejects_bad_dims(B, dims, code):
    with pytest.raises(B.MoeError) as e:
        B.moe_workspace_bytes(B.Dims(*dims))
    assert B.moe_status_string(e.value.status) == code


def test_workspace_grows_with_tokens(B):
    a = B.moe_workspace_bytes(B.Dims(4, 2048, 512, 512, 10, 48))
    b = B.moe_workspace_bytes(B.Dims(8192, 2048, 512, 512, 10, 1))
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0


def _d(B):
    return B.Dims(8, 512, 256, 32, 4, 1)


def test_route_validation(B):
    d = ctypes.byref(_d(B))
    fake = 1 << 20  # an aligned non-null address; never dereferenced on these paths
    # neither router matrix nor logits
    assert B.raw_status("moe_route", d, fake, None, None, fake, None, fake, fake, fake, None) == B.MOE_ERR_ARG
    # both
    assert B.raw_status("moe_route", d, fake, fake, fake, fake, fake, fake, fake, fake, None) == B.MOE_ERR_ARG
    # router matrix without logits_out
    assert B.raw_status("moe_route", d, fake, fake, None, fake, None, fake, fake, fake, None) == B.MOE_ERR_ARG
    # NULL x
    assert B.raw_status("moe_route", d, None, None, fake, fake, None, fake, fake, fake, None) == B.MOE_ERR_ARG
    # misaligned x
    assert B.raw_status("moe_route", d, fake + 2, None, fake, fake, None, fake, fake, fake, None) == B.MOE_ERR_ALIGN


def test_group_validation(B):
    dims = _d(B)
    d = ctypes.byref(dims)
    fake = 1 << 20
    need = B.moe_workspace_bytes(dims)
    args = [fake, fake, 4, fake, fake, fake, fake, fake, fake]
    assert B.raw_status("moe_group", d, 0, *args, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert B.raw_status("moe_group", d, 1, *args, need, None) == B.MOE_ERR_ARG        # layer >= L
    assert B.raw_status("moe_group", d, -1, *args, need, None) == B.MOE_ERR_ARG
    bad = list(args)
    bad[0] = None
    assert B.raw_status("moe_group", d, 0, *bad, need, None) == B.MOE_ERR_ARG


def test_ffn_validation(B):
    dims = _d(B)
    d = ctypes.byref(dims)
    fake = 1 << 20
    lay = B.moe_blob_layout_init(512, 256)
    need = B.moe_workspace_bytes(dims)
    ok_args = (fake, fake, 1 << 30, ctypes.byref(lay), fake, fake, fake, fake, fake, fake, fake, need, None)
    wrong = B.moe_blob_layout_init(512, 512)
    bad_layout = list(ok_args)
    bad_layout[3] = ctypes.byref(wrong)
    assert B.raw_status("moe_expert_ffn", d, *bad_layout) == B.MOE_ERR_ARG
    short_ws = list(ok_args)
    short_ws[11] = need - 256
    assert B.raw_status("moe_expert_ffn", d, *short_ws) == B.MOE_ERR_WORKSPACE
    unaligned_pool = list(ok_args)
    unaligned_pool[1] = fake + 8
    assert B.raw_status("moe_expert_ffn", d, *unaligned_pool) == B.MOE_ERR_ALIGN
    # the staged form rejects a stage mask outside 1..3 before anything else,
    # and validates the rest like moe_expert_ffn
    for stages in (0, 4, -1):
        assert B.raw_status("moe_expert_ffn_stages", d, *ok_args[:-1], stages, None, None, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_expert_ffn_stages", d, *short_ws[:-1], 1, None, None, None) == B.MOE_ERR_WORKSPACE
    assert B.raw_status("moe_expert_ffn_stages", d, *unaligned_pool[:-1], 2, None, None, None) == B.MOE_ERR_ALIGN


def test_route_group_ffn_validation(B):
    """moe_route_group_ffn validates like moe_route_group and
    moe_expert_ffn_stages, and takes stages 1 or 3 only."""
    dims = _d(B)
    d = ctypes.byref(dims)
    fake = 1 << 20
    lay = B.moe_blob_layout_init(512, 256)
    need = B.moe_workspace_bytes(dims)
    ok = [0, fake, None, fake, fake, None, fake, fake, fake, fake, 4, fake, fake, fake, fake, fake, 1 << 30,
          ctypes.byref(lay), fake, fake, fake, fake, need, 3, None, None, None]

    def st(i, v):
        a = list(ok)
        a[i] = v
        return B.raw_status("moe_route_group_ffn", d, *a)
    for stages in (0, 2, 4, -1):
        assert st(23, stages) == B.MOE_ERR_ARG
    assert st(3, None) == B.MOE_ERR_ARG                         # neither router matrix nor logits
    assert st(2, fake) == B.MOE_ERR_ARG                         # both
    assert st(0, 1) == B.MOE_ERR_ARG                            # layer >= L
    assert st(22, need - 256) == B.MOE_ERR_WORKSPACE
    assert st(17, ctypes.byref(B.moe_blob_layout_init(512, 512))) == B.MOE_ERR_ARG
    assert st(15, fake + 8) == B.MOE_ERR_ALIGN                  # pool
    assert st(18, None) == B.MOE_ERR_ARG                        # h


def test_route_group_ffn_mx_validation(B):
    """moe_route_group_ffn_mx validates like moe_route_group and
    moe_expert_ffn_mx (the MX layout and workspace included), and takes
    stages 1 or 3 only."""
    dims = _d(B)
    d = ctypes.byref(dims)
    fake = 1 << 20
    lay = B.moe_blob_layout_init_mx(512, 256)
    need = B.moe_workspace_bytes(dims)
    need_mx = B.moe_mx_workspace_bytes(dims)
    ok = [0, fake, None, fake, fake, None, fake, fake, fake, fake, 4, fake, fake, fake, fake, fake, 1 << 30,
          ctypes.byref(lay), fake, fake, fake, fake, need, fake, need_mx, 3, None, None, None]

    def st(i, v):
        a = list(ok)
        a[i] = v
        return B.raw_status("moe_route_group_ffn_mx", d, *a)
    for stages in (0, 2, 4, -1):
        assert st(25, stages) == B.MOE_ERR_ARG
    assert st(3, None) == B.MOE_ERR_ARG                         # neither router matrix nor logits
    assert st(0, 1) == B.MOE_ERR_ARG                            # layer >= L
    assert st(22, need - 256) == B.MOE_ERR_WORKSPACE
    assert st(24, need_mx - 256) == B.MOE_ERR_WORKSPACE         # MX workspace
    assert st(17, ctypes.byref(B.moe_blob_layout_init(512, 256))) == B.MOE_ERR_ARG   # an NVFP4 layout
    assert st(23, fake + 16) == B.MOE_ERR_ALIGN                 # mx_ws
    assert st(23, None) == B.MOE_ERR_ARG
    assert st(18, None) == B.MOE_ERR_ARG                        # h


@pytest.mark.parametrize("H,I", [(128, 128), (256, 128), (2048, 512), (4096, 2048), (384, 640), (16384, 128)])
def test_mx_blob_layout_matches_oracle(B, H, I):
    lay = B.moe_blob_layout_init_mx(H, I)
    ref = O.mx_blob_layout(H, I)
    assert tuple(lay.off_codes) == ref.off_codes and tuple(lay.off_scales) == ref.off_scales
    assert lay.blob_bytes == ref.blob_bytes == lay.off_globals and lay.slot_stride == ref.slot_stride
    # the codes sit where the NVFP4 blob puts them
    assert tuple(lay.off_codes) == tuple(B.moe_blob_layout_init(H, I).off_codes)


@pytest.mark.parametrize("H,I", [(96, 128), (128, 160), (64, 64), (16512, 128)])
def test_mx_blob_layout_rejects_widths_off_128(B, H, I):
    with pytest.raises(B.MoeError) as e:
        B.moe_blob_layout_init_mx(H, I)
    assert e.value.status == B.MOE_ERR_SHAPE


def test_mx_workspace_matches_documented_layout(B):
    for dims in [B.Dims(64, 256, 128, 8, 2), B.Dims(8192, 2048, 512, 512, 10), B.Dims(3, 384, 640, 4, 4)]:
        assert B.moe_mx_workspace_bytes(dims) == B.MxWorkspace(dims).total


def test_mx_ffn_validation(B):
    """Rejected before any device work: an NVFP4 layout, a short MX workspace
    (for the GEMM and for the decode layout), an unaligned one, a bad stage mask."""
    fake = 1 << 20
    dims = B.Dims(64, 256, 128, 8, 2)               # T k = 128 = 16 E: the GEMM path
    d = ctypes.byref(dims)
    lay = B.moe_blob_layout_init_mx(256, 128)
    need = B.moe_workspace_bytes(dims)
    need_mx = B.moe_mx_workspace_bytes(dims)
    ok = [fake, fake, 1 << 30, ctypes.byref(lay), fake, fake, fake, fake, fake, fake, fake, need, fake, need_mx, 3,
          None, None, None]

    def st(args, dd=d):
        return B.raw_status("moe_expert_ffn_mx", dd, *args)
    small = B.Dims(4, 256, 128, 64, 4)              # T k = 16 < 16 E: the decode layout
    small_ok = list(ok)
    small_ok[11] = B.moe_workspace_bytes(small)
    small_ok[13] = B.moe_mx_workspace_bytes(small) - 256
    assert st(small_ok, ctypes.byref(small)) == B.MOE_ERR_WORKSPACE
    assert B.MxWorkspace(small).total == B.moe_mx_workspace_bytes(small) and not B.MxWorkspace(small).gemm
    nv = B.moe_blob_layout_init(256, 128)
    assert st(ok[:3] + [ctypes.byref(nv)] + ok[4:]) == B.MOE_ERR_ARG
    assert st(ok[:13] + [need_mx - 256] + ok[14:]) == B.MOE_ERR_WORKSPACE
    assert st(ok[:12] + [fake + 16] + ok[13:]) == B.MOE_ERR_ALIGN     # mx_ws must be 256-byte aligned
    for stages in (0, 4):
        assert st(ok[:14] + [stages] + ok[15:]) == B.MOE_ERR_ARG
    assert B.raw_status("moe_quantize_mxfp8", fake, 4, 48, fake, fake, None) == B.MOE_ERR_SHAPE
    assert B.raw_status("moe_quantize_mxfp8", fake + 8, 4, 64, fake, fake, None) == B.MOE_ERR_ALIGN


def test_combine_and_ring_validation(B):
    d = ctypes.byref(_d(B))
    fake = 1 << 20
    assert B.raw_status("moe_combine", d, None, fake, fake, fake, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_combine", d, fake, fake, fake, fake, fake + 4, None) == B.MOE_ERR_ALIGN
    out = ctypes.c_void_p()
    assert B.raw_status("moe_ring_create", None, fake, 4096, None, ctypes.byref(out)) == B.MOE_ERR_ARG
    assert B.raw_status("moe_ring_create", fake, fake + 1, 4096, None, ctypes.byref(out)) == B.MOE_ERR_ALIGN
    assert B.raw_status("moe_ring_destroy", None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_ring_acquire", None, 0, None) == B.MOE_ERR_ARG


@pytest.mark.parametrize("seed", range(6))
def test_swap_plan_matches_oracle(B, seed):
    """moe_swap_plan (host-pure) against the oracle's hot/cold rule on random
    heats (integers and decayed values, so equal heats and equal gaps occur)
    and residency tables; threshold and cap vary."""
    import numpy as np
    rng = np.random.default_rng(seed)
    L, E = int(rng.integers(1, 6)), int(rng.integers(2, 40))
    heat = rng.integers(0, 12, size=(L, E)).astype(np.float32)
    if seed % 2:
        heat *= np.float32(0.7)
    table = np.where(rng.random((L, E + 1)) < 0.5, np.arange(L * (E + 1)).reshape(L, E + 1), -1).astype(np.int32)
    thr, cap = float(rng.choice([0.0, 1.5, 2.0])), int(rng.choice([0, 3, 96]))
    d = B.Dims(1, 64, 32, E, 1, L)
    got = [tuple(r) for r in B.moe_swap_plan(d, heat, table, thr, cap)]
    assert got == O.swap_plan(heat, table, thr, cap)


def test_noalloc_refuses_dims_beyond_its_static_scratch(B):
    """moe_expert_ffn_mx_noalloc refuses, before any HIP call, dims whose MX
    workspace exceeds the library's 32 MiB static scratch."""
    big = B.Dims(8192, 2048, 512, 512, 10, 1)
    assert B.moe_mx_workspace_bytes(big) > 32 << 20
    assert B.moe_mx_workspace_bytes(B.Dims(4096, 2048, 512, 512, 10, 1)) <= 32 << 20
    lay = B.moe_blob_layout_init_mx(2048, 512)
    ws_bytes = B.moe_workspace_bytes(big)
    p = 1 << 20   # aligned stand-in addresses: validation fails before any of them is used
    rc = B.raw_status("moe_expert_ffn_mx_noalloc", ctypes.byref(big), p, p, lay.slot_stride * 8, ctypes.byref(lay),
                      p, p, p, p, p, p, p, ws_bytes, 3, None)
    assert rc == B.MOE_ERR_WORKSPACE
    assert b"static" in B._lib.moe_last_error()


def test_probe_validation(B):
    """The measurement probes refuse bad arguments before enqueueing anything."""
    fake = 1 << 20
    assert B.raw_status("moe_probe_hbm_read", None, 8192, 64, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_hbm_read", fake, 8192 + 1024, 64, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_hbm_read", fake, 0, 64, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_hbm_read", fake + 4, 8192, 64, fake, None) == B.MOE_ERR_ALIGN
    assert B.raw_status("moe_probe_hbm_read", fake, 8192, 0, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_mfma", 3, 1, 1, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_mfma", 0, 0, 1, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_mfma", 0, 1, 0, fake, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_mfma", 1, 1, 1, None, None) == B.MOE_ERR_ARG
    f = fake
    assert B.raw_status("moe_probe_scaled_mfma", None, f, f, f, 1, 0, f, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_scaled_mfma", f, f, f, f, 1, 0, None, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_scaled_mfma", f, f, f, f, 0, 0, f, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_scaled_mfma", f, f, f, f, (1 << 16) + 1, 0, f, None) == B.MOE_ERR_ARG
    assert B.raw_status("moe_probe_scaled_mfma", f, f, f, f, 1, 2, f, None) == B.MOE_ERR_ARG

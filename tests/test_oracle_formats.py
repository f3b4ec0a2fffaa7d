"""Pins of the oracle's format decoders and rounding (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (golden fixtures), a library routine (torch's float8_e4m3fn and
bfloat16 conversions), closed forms, or brute force."""
import struct

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import moe_oracle as O


def test_e2m1_matches_page_table():
    rows = read_golden("e2m1_table.txt")
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = O.e2m1_decode(codes)
    assert len(codes) == 16
    np.testing.assert_array_equal(got, want)


def test_e4m3fn_exhaustive_vs_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_decode(b)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_packed_row_bytes_page_example():
    g = {r[0]: int(r[1]) for r in read_golden("packed_row_bytes.txt")}
    code_b, scale_b = O.matrix_bytes(1, g["row_values"])
    assert code_b == g["row_code_bytes"] and scale_b == g["row_scale_bytes"]
    assert code_b + scale_b == g["row_bytes"]
    c16, s16 = O.matrix_bytes(g["rows_per_token"], g["row_values"])
    assert c16 + s16 == g["token_packed_bytes"]
    assert g["rows_per_token"] * g["row_values"] * 2 == g["token_bf16_bytes"]


def test_pool_shape_page_estimate():
    g = {r[0]: float(r[1]) for r in read_golden("pool_shape.txt")}
    H, I = int(g["H"]), int(g["I"])
    per_expert = sum(O.matrix_bytes(*O.blob_layout(H, I).matrix_shape(m))[0] for m in range(3))
    total = g["layers"] * g["experts"] * per_expert
    assert abs(total / g["approx_bytes"] - 1.0) <= g["rel_tol"]


def test_blob_layout_hand_computed():
    # H = I = 32: every matrix is 32 x 32 -> 512 code bytes, 64 scale bytes.
    lay = O.blob_layout(32, 32)
    assert lay.off_codes == (0, 512, 1024)
    assert lay.off_scales == (1536, 1792, 2048)
    assert lay.off_globals == 2304 and lay.blob_bytes == 2316 and lay.slot_stride == 4096
    # closed form when every section is already 256-aligned: 27 H I / 16 + 12
    for H, I in [(512, 256), (2048, 512), (4096, 2048)]:
        assert O.blob_layout(H, I).blob_bytes == 27 * H * I // 16 + 12


def _hand_blob():
    """H = I = 32 blob built byte by byte (offsets from the hand computation)."""
    buf = bytearray(4096)
    off_c, off_s, off_g = (0, 512, 1024), (1536, 1792, 2048), 2304
    G = (0.5, 2.0, 0.25)
    for m in range(3):
        struct.pack_into("<f", buf, off_g + 4 * m, G[m])
    # gate row 0: col 0 = code 7 (+6), col 1 = code 0xF (-6), col 2 = code 1 (+0.5), col 3 = code 0xA (-1)
    buf[off_c[0] + 0] = 0x7 | (0xF << 4)
    buf[off_c[0] + 1] = 0x1 | (0xA << 4)
    # gate row 0 scales: block 0 -> 1.0 (0x38), block 1 -> 2^-9 (0x01)
    buf[off_s[0] + 0] = 0x38
    buf[off_s[0] + 1] = 0x01
    # gate row 0, col 16 (block 1): code 6 (+4)
    buf[off_c[0] + 8] = 0x6
    # gate row 5 (stride 16 code bytes, 2 scale bytes): col 31 = code 5 (+3), scale 448 (0x7E)
    buf[off_c[0] + 5 * 16 + 15] = 0x5 << 4
    buf[off_s[0] + 5 * 2 + 1] = 0x7E
    # up row 0: col 0 = code 2 (+1), scale 1.5 (0x3C)
    buf[off_c[1]] = 0x2
    buf[off_s[1]] = 0x3C
    # down row 31: col 30 = code 0xC (-2), scale 0.875 (0x36: e=6, m=6 -> (1+6/8) 2^-1)
    buf[off_c[2] + 31 * 16 + 15] = 0xC
    buf[off_s[2] + 31 * 2 + 1] = 0x36
    return bytes(buf), G


def test_dequant_hand_built_blob():
    blob, G = _hand_blob()
    lay = O.blob_layout(32, 32)
    wg, wu, wd = (O.dequant(blob, lay, m) for m in range(3))
    assert wg[0, 0] == 6 * 1.0 * G[0] and wg[0, 1] == -6 * 1.0 * G[0]    # low nibble = even column
    assert wg[0, 2] == 0.5 * G[0] and wg[0, 3] == -1.0 * G[0]
    assert wg[0, 16] == 4 * 2.0 ** -9 * G[0]                               # block 1 uses scale 1
    assert wg[5, 31] == 3 * 448.0 * G[0]
    assert wu[0, 0] == 1.0 * 1.5 * G[1]
    assert wd[31, 30] == -2 * 0.875 * G[2]
    # every other value is zero
    assert np.count_nonzero(wg) == 6 and np.count_nonzero(wu) == 1 and np.count_nonzero(wd) == 1


def _hand_tiled_blob():
    """H = 544, I = 32 blob, bytes placed by hand from the tiling in include/moe.h.

    gate and up are [32 rows][544 cols]: 2 row blocks of 8*544 = 4352 code bytes
    and 544 scale bytes; 17 chunks, so scale group 0 holds 32 bytes per row and
    group 1 (chunk 16 only) 2 bytes per row.  down is [544 rows][32 cols]: 34
    row blocks of 256 code bytes and 32 scale bytes."""
    lay = O.blob_layout(544, 32)
    buf = bytearray(lay.slot_stride)
    G = (0.5, 2.0, 0.25)
    for m in range(3):
        struct.pack_into("<f", buf, lay.off_globals + 4 * m, G[m])
    cg, cu, cd = lay.off_codes
    sg, su, sd = lay.off_scales
    # gate row 0, col 1: block 0, chunk 0, row 0, byte 0, high nibble: code 9 (-0.5); scale 0 at byte 0
    buf[cg + 0] = 0x9 << 4
    buf[sg + 0] = 0x38
    # gate row 17, col 40: block 1 (4352), chunk 1 (+256), row 1 (+16), byte 4, low nibble: code 7 (+6)
    buf[cg + 4352 + 256 + 16 + 4] = 0x7
    # its scale (b = 2): block 1 (544) + group 0 + row 1 * 32 + 2 -> 1.0
    buf[sg + 544 + 32 + 2] = 0x38
    # gate row 17, col 530: chunk 16 (+4096), row 1 (+16), byte 9, low nibble: code 3 (+1.5)
    buf[cg + 4352 + 4096 + 16 + 9] = 0x3
    # its scale (b = 33): block 1 (544) + group 1 (512) + row 1 * 2 + 1 -> 2.0 (0x40)
    buf[sg + 544 + 512 + 2 + 1] = 0x40
    # up row 31, col 543: the last code byte of the section, high nibble: code 5 (+3)
    buf[cu + 4352 + 4096 + 15 * 16 + 15] = 0x5 << 4
    # its scale (b = 33): 544 + 512 + row 15 * 2 + 1, the last scale byte -> 448 (0x7E)
    buf[su + 544 + 512 + 30 + 1] = 0x7E
    # down row 543, col 31: block 33 (33 * 256), chunk 0, row 15 (+240), byte 15, high nibble: code 0xC (-2)
    buf[cd + 33 * 256 + 240 + 15] = 0xC << 4
    # its scale (b = 1): block 33 (33 * 32) + row 15 * 2 + 1 -> 0.875 (0x36)
    buf[sd + 33 * 32 + 30 + 1] = 0x36
    return bytes(buf), lay, G


def test_dequant_hand_built_tiled_blob():
    blob, lay, G = _hand_tiled_blob()
    assert lay.off_codes == (0, 8704, 17408) and lay.off_scales[0] == 26112
    wg, wu, wd = (O.dequant(blob, lay, m) for m in range(3))
    assert wg.shape == (32, 544) and wd.shape == (544, 32)
    assert wg[0, 1] == -0.5 * G[0]
    assert wg[17, 40] == 6 * 1.0 * G[0]
    assert wg[17, 530] == 1.5 * 2.0 * G[0]
    assert wu[31, 543] == 3 * 448.0 * G[1]
    assert wd[543, 31] == -2 * 0.875 * G[2]
    assert np.count_nonzero(wg) == 3 and np.count_nonzero(wu) == 1 and np.count_nonzero(wd) == 1
    # the up and down entries are the last byte of their sections
    assert blob[lay.off_codes[1] + 8703] == 0x50 and blob[lay.off_scales[1] + 1087] == 0x7E
    assert blob[lay.off_codes[2] + 8703] == 0xC0 and blob[lay.off_scales[2] + 1087] == 0x36


def test_bf16_round_vs_torch_fp32_inputs():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),     # bf16 subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 3.3895e38, 3.4e38, -3.4e38, 1e-45], dtype=np.float32),
    ])
    # exact ties: bf16 value plus half a unit in the last place (both even and odd neighbours)
    base = (rng.integers(0x3000, 0x5000, 4000, dtype=np.uint32) << 16).view(np.float32)
    ties = (base.view(np.uint32) + 0x8000).view(np.float32)
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_fp64_inputs_brute_force():
    grid = O.bf16_bits_to_f64(np.arange(0, 0x7F80, dtype=np.uint16))   # all finite non-negative bf16
    rng = np.random.default_rng(2)
    v = np.abs(np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                               rng.standard_normal(500) * 1e-39]))
    got = O.bf16_round(v)
    idx = np.searchsorted(grid, v)
    for x, g, i in zip(v, got, idx):
        lo, hi = grid[max(i - 1, 0)], grid[min(i, len(grid) - 1)]
        if grid[min(i, len(grid) - 1)] == x:
            want = x
        else:
            dlo, dhi = x - lo, hi - x
            if dlo < dhi:
                want = lo
            elif dhi < dlo:
                want = hi
            else:  # tie: even bit pattern
                want = lo if (i - 1) % 2 == 0 else hi
        assert g == want, (x, g, want)


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(O.bf16_bits_to_f64(bits)), bits)

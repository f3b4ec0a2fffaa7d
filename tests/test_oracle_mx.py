"""Pins of the oracle's MX formats (CPU only).

The reading is the OCP Microscaling one: E8M0 block scales over 32 values, E2M1
weight elements with no global scale, and activations quantised to MXFP8 (E4M3
elements, shared exponent floor(log2 amax) - 8, nearest-even rounding that
saturates at 448).  Each test checks the oracle against something other than
itself:
- torch's float8_e8m0fnu and float8_e4m3fn conversions;
- hand-derived values and closed-form bounds;
- a blob placed byte by byte from the layout formula;
- compositions with the NVFP4 FFN, which has its own pins."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def test_e8m0_exhaustive_vs_torch_and_closed_form():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.e8m0_decode(b)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert all(got[i] == math.ldexp(1.0, i - 127) for i in range(255))


def _finite_e4m3():
    v = O.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    return np.unique(v[~np.isnan(v)])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200000))
    v = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    vals = _finite_e4m3()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)      # every tie, exact in fp32
    v = np.concatenate([v, vals.astype(np.float32), mids, -mids, np.float32([0.0, 448.0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3fn_encode(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_hand_values():
    cases = {1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, 3.0: 0x44, -3.0: 0xC4,
             2.0 ** -9: 0x01, 3 * 2.0 ** -10: 0x02, 2.0 ** -10: 0x00,
             448.0: 0x7E, 449.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE}
    for v, code in cases.items():
        assert int(O.e4m3fn_encode(v)) == code, v


def test_mxfp8_hand_examples():
    v = np.zeros((4, 64))
    v[0, 0] = 448.0                       # amax 448: 2^8 <= 448 < 2^9 -> X = 1
    v[1, 0], v[1, 1] = 500.0, 1.0         # X = 1, 500 saturates to 448
    v[2, 0], v[2, 1] = 0.75, 1.0 / 3      # X = 2^-9: 1/3 -> 170.67 -> 176
    v[3, 32] = -2.0 ** -20                # one value; the first block of the row is zero
    codes, sc, q = O.mxfp8_quantize(v)
    assert sc[0, 0] == 127 and q[0, 0] == 448.0
    assert sc[1, 0] == 127 and q[1, 0] == 448.0 and q[1, 1] == 1.0
    assert sc[2, 0] == 127 - 9 and q[2, 0] == 0.75 and q[2, 1] == 176 * 2.0 ** -9
    assert sc[3, 0] == 0 and not codes[3, :32].any() and not q[3, :32].any()
    assert sc[3, 1] == 127 - 28 and q[3, 32] == -2.0 ** -20 and codes[3, 32] == 0xF8   # -256 * 2^-28: exponent field 15, mantissa 0


def test_mxfp8_exponent_clamps():
    v = np.zeros((2, 32))
    v[0, 0] = 2.0 ** -140                 # floor(log2) - 8 = -148 < -127
    v[1, 0] = 2.0 ** 130                  # 122, inside the range
    _, sc, q = O.mxfp8_quantize(v)
    assert sc[0, 0] == 0 and q[0, 0] == 0.0          # 2^-140 / 2^-127 = 2^-13 < half of 2^-9
    assert sc[1, 0] == 127 + 122 and q[1, 0] == 2.0 ** 130


def test_mxfp8_block_bounds():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))
    v *= np.exp2(rng.uniform(-6, 0, v.shape))        # wide range inside each block
    codes, sc, q = O.mxfp8_quantize(v)
    for n in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk, qb = v[n, 32 * b:32 * b + 32], q[n, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            m, e = math.frexp(amax)                   # amax = m 2^e, m in [0.5, 1)
            X = math.ldexp(1.0, e - 1 - 8)
            assert sc[n, b] == e - 1 - 8 + 127
            assert 256 * X <= np.abs(qb).max() <= 448 * X
            ok = np.abs(blk) <= 448 * X
            err = np.abs(blk - qb)
            assert np.all(err[ok] <= np.maximum(2.0 ** -4 * np.abs(blk[ok]), 2.0 ** -10 * X))
            assert np.all(np.abs(qb[~ok]) == 448 * X)
            assert np.all(np.sign(qb) * np.sign(blk) >= 0)


def test_mx_blob_layout_hand_computed():
    lay = O.mx_blob_layout(256, 128)
    # gate/up [128 x 256] and down [256 x 128]: 16384 code bytes and 1024 scale bytes each
    assert lay.off_codes == (0, 16384, 32768)
    assert lay.off_scales == (49152, 50176, 51200)
    assert lay.blob_bytes == 52224 and lay.slot_stride == 53248
    with pytest.raises(AssertionError):
        O.mx_blob_layout(256, 96)


def _place(blob, off_c, off_s, codes, sbytes):
    """Byte-by-byte placement from the layout formula: row n, column c's nibble
    (low nibble = even column) at 8K(n//16) + 256(c//32) + 16(n%16) + (c%32)//2;
    the scale of (n, block b) at (n//16)(K/2) + 64(b//4) + 4(n%16) + b%4."""
    R, K = codes.shape
    for n in range(R):
        for c in range(0, K, 2):
            pos = off_c + 8 * K * (n // 16) + 256 * (c // 32) + 16 * (n % 16) + (c % 32) // 2
            blob[pos] = int(codes[n, c]) | (int(codes[n, c + 1]) << 4)
        for b in range(K // 32):
            blob[off_s + (n // 16) * (K // 2) + 64 * (b // 4) + 4 * (n % 16) + b % 4] = int(sbytes[n, b])


def test_mx_dequant_hand_built_blob():
    H, I = 256, 128
    lay = O.mx_blob_layout(H, I)
    rng = np.random.default_rng(3)
    blob = np.zeros(lay.slot_stride, np.uint8)
    want = []
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for m, (R, K) in enumerate(((I, H), (I, H), (H, I))):
        codes = rng.integers(0, 16, (R, K))
        sbytes = rng.integers(100, 150, (R, K // 32))
        _place(blob, lay.off_codes[m], lay.off_scales[m], codes, sbytes)
        val = np.array([[(-1.0 if c & 8 else 1.0) * e2m1[c & 7] for c in row] for row in codes])
        want.append(val * np.repeat(np.exp2(sbytes - 127.0), 32, axis=1))
    for m in range(3):
        np.testing.assert_array_equal(O.mx_dequant(blob, lay, m, H, I), want[m])


def _q(v):
    return O.mxfp8_quantize(v)[2]


def test_expert_ffn_mx_quantises_x():
    """x = 1/3 in a block led by 0.75 meets the weights as 176 * 2^-9."""
    rng = np.random.default_rng(1)
    H, I = 64, 32
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((I, H), (I, H), (H, I)))
    x = np.full((1, H), 1.0 / 3)
    x[0, 0] = x[0, 32] = 0.75
    x_hand = np.full((1, H), 176 * 2.0 ** -9)
    x_hand[0, 0] = x_hand[0, 32] = 0.75
    a, b = O.expert_ffn_mx(x, wg, wu, wd), O.expert_ffn_mx(x_hand, wg, wu, wd)
    np.testing.assert_array_equal(a.y, b.y)
    np.testing.assert_array_equal(a.h, b.h)
    assert not np.array_equal(O.expert_ffn(x, wg, wu, wd).h, a.h)


def test_expert_ffn_mx_down_input_is_quantised_bf16_h():
    """With W_d = identity, Y is the MXFP8 value of h = bf16(silu(g) u), g and u
    taken from the quantised x through the pinned NVFP4 FFN."""
    rng = np.random.default_rng(2)
    H = I = 128
    wg, wu = rng.standard_normal((I, H)) * 0.1, rng.standard_normal((I, H)) * 0.1
    x = rng.standard_normal((5, H))
    eye = np.eye(H)
    mx = O.expert_ffn_mx(x, wg, wu, eye)
    nv = O.expert_ffn(_q(x), wg, wu, eye)
    np.testing.assert_array_equal(mx.h, nv.h)
    np.testing.assert_array_equal(mx.y, _q(nv.h))          # E4M3 * 2^s values are bf16-exact
    assert not np.array_equal(mx.y, nv.y)


def test_expert_ffn_mx_close_to_unquantised():
    """Quantisation error stays inside the E4M3 bound: |x - q(x)| <= 2^-4 |x|
    (normal range) propagates to well under 10 % of the output norm."""
    rng = np.random.default_rng(4)
    H, I = 256, 128
    wg, wu, wd = (rng.standard_normal(s) / math.sqrt(s[1]) for s in ((I, H), (I, H), (H, I)))
    x = rng.standard_normal((16, H))
    mx, nv = O.expert_ffn_mx(x, wg, wu, wd), O.expert_ffn(x, wg, wu, wd)
    rel = np.linalg.norm(mx.y_pre - nv.y_pre) / np.linalg.norm(nv.y_pre)
    assert 1e-4 < rel < 0.1

"""Pins of the oracle's expert FFN, combine and whole layer (CPU only).

The expert FFN is checked against a textbook dense FFN computed with torch in
float64 on weights decoded by an independent route (torch's float8_e4m3fn for
the scales, the page's E2M1 table for the codes).  The layer is checked against
closed forms: k = E with uniform logits is the dense mixture, k = 1 is one
dense FFN, tokens permute bit-exactly, and dropping experts changes the output
by exactly their weighted terms."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from conftest import read_golden
from oracle import moe_oracle as O
from synth import Config, HostGen


PIN = Config(cfg_id=9, name="pin", T=6, H=64, I=32, E=5, k=2, L=1, router="matrix")


def _indep_decode(blob, H, I):
    """Decode a blob without the oracle's decoders (layout offsets recomputed here)."""
    table = {int(r[0]): float(r[1]) for r in read_golden("e2m1_table.txt")}
    lut = torch.tensor([table[c] for c in range(16)], dtype=torch.float64)
    b = torch.from_numpy(np.frombuffer(bytes(blob), dtype=np.uint8).copy())
    align = lambda v: (v + 255) // 256 * 256
    shapes = [(I, H), (I, H), (H, I)]
    off, oc, osc = 0, [], []
    for r, K in shapes:
        oc.append(off)
        off = align(off + r * K // 2)
    for r, K in shapes:
        osc.append(off)
        off = align(off + r * K // 16)
    glob = b[off:off + 12].numpy().view(np.float32).astype(np.float64)
    mats = []
    for m, (r, K) in enumerate(shapes):
        # byte positions from the 16-row block tiling, one index per element
        n = torch.arange(r).view(r, 1)
        c = torch.arange(K // 2).view(1, K // 2)
        cpos = (n // 16) * 8 * K + 256 * (c // 16) + 16 * (n % 16) + c % 16
        codes = b[oc[m] + cpos].to(torch.int64)
        vals = torch.stack([lut[codes & 15], lut[codes >> 4]], dim=-1).reshape(r, K)
        sb = torch.arange(K // 16).view(1, K // 16)
        g = sb // 32
        per_row = torch.clamp(K // 16 - 32 * g, max=32)
        spos = (n // 16) * K + 512 * g + per_row * (n % 16) + sb - 32 * g
        sc = b[osc[m] + spos].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
        mats.append(vals * sc.repeat_interleave(16, dim=1) * glob[m])
    return mats


def _textbook_ffn(x, wg, wu, wd):
    """down(silu(gate x) * (up x)) with the two bf16 rounding points, torch float64."""
    xt = torch.as_tensor(x, dtype=torch.float64)
    h_pre = F.silu(xt @ wg.T) * (xt @ wu.T)
    h = torch.as_tensor(O.bf16_round(h_pre.numpy()))
    y_pre = h @ wd.T
    return h_pre.numpy(), h.numpy(), y_pre.numpy()


@pytest.fixture(scope="module")
def pin_inputs(hostgen):
    lay = O.blob_layout(PIN.H, PIN.I)
    blobs = {e: hostgen.expert_blob(PIN, 0, e, lay) for e in range(PIN.E + 1)}
    x = hostgen.x(PIN, 0)
    wr = hostgen.w_router(PIN, 0)
    wsg = hostgen.w_shared_gate(PIN, 0) * 10   # a gate far from 0.5 so the sigma term matters
    return lay, blobs, x, wr, wsg


def test_expert_ffn_vs_textbook(pin_inputs):
    lay, blobs, x_bits, _, _ = pin_inputs
    x = O.bf16_bits_to_f64(x_bits)
    for e in (0, 3, PIN.E):
        wg, wu, wd = _indep_decode(blobs[e], PIN.H, PIN.I)
        ours = O.expert_ffn(x, *(O.dequant(blobs[e], lay, m) for m in range(3)))
        h_pre, h, y_pre = _textbook_ffn(x, wg, wu, wd)
        np.testing.assert_allclose(ours.h_pre, h_pre, rtol=1e-12, atol=1e-300)
        np.testing.assert_array_equal(ours.h, h)
        np.testing.assert_allclose(ours.y_pre, y_pre, rtol=1e-12, atol=1e-300)
        np.testing.assert_array_equal(ours.y, O.bf16_round(y_pre))
        # the two projections are not interchangeable: swapping gate and up must change h
        swapped = F.silu(torch.as_tensor(x) @ wu.T) * (torch.as_tensor(x) @ wg.T)
        assert not np.allclose(swapped.numpy(), h_pre, rtol=1e-3)


def test_k_equals_E_uniform_is_dense_mixture(pin_inputs):
    lay, blobs, x_bits, _, wsg = pin_inputs
    E = PIN.E
    logits = np.zeros((PIN.T, E), np.float32)
    r = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, E, E, wsg, logits=logits)
    assert np.array_equal(r.ids, np.tile(np.arange(E, dtype=np.int32), (PIN.T, 1)))
    np.testing.assert_allclose(r.w, 1.0 / E, rtol=1e-15)
    x = O.bf16_bits_to_f64(x_bits)
    dense = np.zeros((PIN.T, PIN.H))
    for e in range(E):
        dense += (1.0 / E) * O.bf16_round(_textbook_ffn(x, *_indep_decode(blobs[e], PIN.H, PIN.I))[2])
    sig = 1.0 / (1.0 + np.exp(-(x @ wsg.astype(np.float64))))
    dense += sig[:, None] * O.bf16_round(_textbook_ffn(x, *_indep_decode(blobs[E], PIN.H, PIN.I))[2])
    np.testing.assert_allclose(r.y_pre, dense, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(r.y, O.bf16_round(dense))


def test_k1_routed_row_is_dense_ffn(pin_inputs):
    lay, blobs, x_bits, wr, wsg = pin_inputs
    r = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, PIN.E, 1, wsg, w_router=wr)
    assert np.all(r.w == 1.0)
    x = O.bf16_bits_to_f64(x_bits)
    for t in range(PIN.T):
        e = int(r.ids[t, 0])
        p = int(r.groups.inv_perm[t])
        want = O.bf16_round(_textbook_ffn(x[t:t + 1], *_indep_decode(blobs[e], PIN.H, PIN.I))[2])[0]
        np.testing.assert_array_equal(r.y_rows[p], want)


def test_token_permutation_is_bit_exact(pin_inputs):
    lay, blobs, x_bits, wr, wsg = pin_inputs
    a = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, PIN.E, PIN.k, wsg, w_router=wr)
    pi = np.random.default_rng(6).permutation(PIN.T)
    b = O.moe_layer(x_bits[pi], lambda e: blobs[e], PIN.H, PIN.I, PIN.E, PIN.k, wsg, w_router=wr)
    assert np.array_equal(b.ids, a.ids[pi])
    assert np.array_equal(b.y, a.y[pi])
    assert np.array_equal(b.w, a.w[pi])


def test_dropping_experts_changes_output_by_their_terms(pin_inputs):
    """[Strata] "少算这些专家，会付出什么代价？": skipped output - full output
    = -sum over skipped experts of w_i E_i(x); the kept weights are not renormalised."""
    lay, blobs, x_bits, wr, wsg = pin_inputs
    r = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, PIN.E, PIN.k, wsg, w_router=wr)
    T, k = PIN.T, PIN.k
    yr = np.stack([np.stack([r.y_rows[int(r.groups.inv_perm[t * k + j])] for j in range(k)]) for t in range(T)])
    ysh = np.stack([r.y_rows[T * k + t] for t in range(T)])
    full, _ = O.combine(yr, r.w, r.sigma, ysh)
    np.testing.assert_array_equal(full, r.y_pre)
    skip = np.zeros_like(r.w, dtype=bool)
    skip[:, k - 1] = True                       # drop the last-ranked slot of every token
    w_skip = np.where(skip, 0.0, r.w)
    skipped, _ = O.combine(yr, w_skip, r.sigma, ysh)
    delta = -np.einsum("tj,tjh->th", np.where(skip, r.w, 0.0), yr)
    np.testing.assert_allclose(skipped - full, delta, rtol=1e-12, atol=1e-12)
    # the shared term enters with weight sigma, outside the softmax
    no_shared, _ = O.combine(yr, r.w, np.zeros(T), ysh)
    np.testing.assert_allclose(full - no_shared, r.sigma[:, None] * ysh, rtol=1e-12, atol=1e-12)


def test_sampled_tokens_match_full_layer(pin_inputs):
    lay, blobs, x_bits, wr, wsg = pin_inputs
    full = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, PIN.E, PIN.k, wsg, w_router=wr)
    sub = O.moe_layer(x_bits, lambda e: blobs[e], PIN.H, PIN.I, PIN.E, PIN.k, wsg, w_router=wr, tokens=[4, 1])
    assert list(sub.tokens) == [1, 4]
    assert np.array_equal(sub.y, full.y[[1, 4]])
    for p, v in sub.y_rows.items():
        assert np.array_equal(v, full.y_rows[p])

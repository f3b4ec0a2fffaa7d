"""Pins of the oracle's router, top-k, weights, shared gate and grouping (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from conftest import read_golden
from oracle import moe_oracle as O


def _fp32_nearest(fr: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (brute force over neighbours)."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.array(v).view(np.uint32)) & 1))
    return np.float32(best)


def test_router_logits_exact_rational():
    rng = np.random.default_rng(3)
    T, H, E = 5, 24, 7
    x = O.bf16_round(rng.standard_normal((T, H)))
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    got = O.router_logits(x, w)
    assert got.dtype == np.float32
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(w[h, e])) for h in range(H))
            assert got[t, e] == _fp32_nearest(exact)


def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]


@pytest.mark.parametrize("E,k", [(8, 3), (32, 4), (17, 17), (5, 1)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 64
    cases = [rng.integers(-3, 3, (T, E)).astype(np.float32),        # heavy ties
             rng.standard_normal((T, E)).astype(np.float32),
             np.zeros((2, E), np.float32)]                           # all equal
    for lg in cases:
        ids = O.topk(lg, k)
        for t in range(lg.shape[0]):
            assert list(ids[t]) == _brute_topk(lg[t].tolist(), k)


def test_topk_weights_closed_forms():
    lg = np.array([[np.log(3.0), 0.0, -5.0]], dtype=np.float64)
    ids = O.topk(lg.astype(np.float32), 2)
    assert list(ids[0]) == [0, 1]
    w = O.topk_weights(np.array([[np.log(3.0), 0.0, -5.0]]), ids)
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=0, atol=1e-15)
    # k = 1 -> weight exactly 1
    assert O.topk_weights(lg, np.array([[2]]))[0, 0] == 1.0


def test_topk_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((50, 40)).astype(np.float32)
    ids = O.topk(lg, 6)
    w = O.topk_weights(lg, ids)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)          # slot order = descending weight


def test_shared_gate_closed_form_and_library():
    x = np.zeros((1, 16))
    assert O.shared_gate(x, np.ones(16))[0] == 0.5
    rng = np.random.default_rng(5)
    x = O.bf16_round(rng.standard_normal((9, 32)))
    wsg = rng.standard_normal(32) * 0.3
    z = np.array([float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, wsg))) for row in x])
    np.testing.assert_allclose(O.shared_gate(x, wsg), scipy.special.expit(z), rtol=1e-14)
    assert np.all(O.shared_gate(x, wsg)[z > 0] > 0.5)   # sign of the exponent


def test_grouping_page_example():
    g = {r[0]: [int(v) for v in r[1:]] for r in read_golden("grouping_example.txt")}
    E, k = g["E"][0], g["k"][0]
    ids = np.array(g["ids"], dtype=np.int32).reshape(-1, k)
    grp = O.group(ids, E)
    e = g["expect_group"][0]
    assert grp.offsets[e + 1] - grp.offsets[e] == g["expect_count"][0]
    nonempty = [i for i in range(E) if grp.offsets[i + 1] > grp.offsets[i]]
    assert nonempty == [e]
    rows = grp.perm[grp.offsets[e]:grp.offsets[e + 1]]
    assert [f // k for f in rows] == g["expect_tokens"]          # three inputs, in token order
    assert sorted(grp.inv_perm.tolist()) == list(range(len(rows)))  # three output positions


@pytest.mark.parametrize("T,k,E", [(13, 3, 7), (40, 10, 64), (1, 1, 1), (6, 4, 4)])
def test_grouping_brute_force(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    grp = O.group(ids, E)
    flat = ids.reshape(-1)
    want_perm = sorted(range(T * k), key=lambda f: (flat[f], f))
    assert grp.perm.tolist() == want_perm
    counts = np.bincount(flat, minlength=E)
    assert grp.offsets[:E + 1].tolist() == [0] + np.cumsum(counts).tolist()
    assert grp.offsets[E + 1] == T * k + T
    assert np.array_equal(grp.perm[grp.inv_perm], np.arange(T * k))

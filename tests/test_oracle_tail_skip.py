"""Pins of the route tail-skip variant in the oracle (CPU only).

[Strata] "少算这些专家，会付出什么代价？" and the skip-condition passage just before
it: with the default threshold 7 (ranks from zero), a non-resident expert that
every token of the window ranks 8th to 10th is skipped; one token ranking it
in its top seven keeps it; resident experts are kept; the other weights are
not renormalised, so the output moves by exactly -sum of the skipped
w_i E_i(x).  The rule is checked on hand-built windows, the layer against that
closed form written out from the unskipped layer's own rows."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import Config

PIN = Config(cfg_id=9, name="pin", T=6, H=64, I=32, E=5, k=2, L=1, router="matrix")


def _window(ranks, E=32, k=10, expert=17):
    """ids [len(ranks), k]: token t picks `expert` at slot ranks[t] (None: not at
    all) and fills its other slots with resident experts 0, 1, 2, ..."""
    ids = np.zeros((len(ranks), k), np.int32)
    for t, r in enumerate(ranks):
        others = iter(e for e in range(E) if e != expert)
        for j in range(k):
            ids[t, j] = expert if j == r else next(others)
    return ids


def _resident(E=32, not_resident=(17,)):
    m = np.ones(E, bool)
    m[list(not_resident)] = False
    return m


@pytest.mark.parametrize("ranks,R,skipped", [
    ((7, 8, 9), 7, True),       # every token ranks it 8th-10th: skipped
    ((7, 8, 6), 7, False),      # one token ranks it 7th: kept
    ((9, None, None), 7, True),  # picked by one token only, at 10th
    ((7, 8, 9), 8, False),      # threshold 8: the token ranking it 8th keeps it
    ((7, 8, 9), 0, False),      # threshold 0: no skipping
    ((None, None, None), 7, False),  # not picked: nothing to skip
])
def test_rule_on_hand_built_windows(ranks, R, skipped):
    ids = _window(ranks)
    got = O.tail_skip(ids, _resident(), R)
    assert bool(got[17]) == skipped
    assert not got[np.arange(32) != 17].any()   # resident experts are never skipped


def test_resident_expert_is_kept():
    ids = _window((7, 8, 9))
    assert not O.tail_skip(ids, _resident(not_resident=()), 7).any()


@pytest.fixture(scope="module")
def skip_case(hostgen):
    lay = O.blob_layout(PIN.H, PIN.I)
    blobs = {e: hostgen.expert_blob(PIN, 0, e, lay) for e in range(PIN.E + 1)}
    x = hostgen.x(PIN, 0)
    wsg = hostgen.w_shared_gate(PIN, 0) * 10
    lg = np.random.default_rng(3).normal(size=(PIN.T, PIN.E)).astype(np.float32)
    lg[:, 3] = lg[:, 4] = -9.0
    # expert 4: second for tokens 0-2, unpicked otherwise; expert 3: first for
    # token 5 and second for token 4
    for t in range(3):
        lg[t, 4] = lg[t, :3].max() - 0.25
    lg[5, 3] = lg[5].max() + 0.5
    lg[4, 3] = lg[4, :3].max() - 0.25
    return blobs, x, wsg, lg


def test_layer_moves_by_the_skipped_terms(skip_case):
    blobs, x, wsg, lg = skip_case
    T, k, E = PIN.T, PIN.k, PIN.E
    full = O.moe_layer(x, lambda e: blobs[e], PIN.H, PIN.I, E, k, wsg, logits=lg)
    resident = np.array([True, True, True, False, False])
    mask = O.tail_skip(full.ids, resident, 1)
    assert list(mask) == [False, False, False, False, True]   # 3 is first for token 5
    skip = O.moe_layer(x, lambda e: blobs[e], PIN.H, PIN.I, E, k, wsg, logits=lg, skip=mask)
    assert np.array_equal(skip.ids, full.ids) and np.array_equal(skip.w, full.w)  # no renormalisation
    delta = np.zeros((T, PIN.H))
    for t in range(T):
        for j in range(k):
            if mask[full.ids[t, j]]:
                delta[t] -= full.w[t, j] * full.y_rows[int(full.groups.inv_perm[t * k + j])]
    assert np.abs(delta).max() > 0
    np.testing.assert_allclose(skip.y_pre - full.y_pre, delta, rtol=1e-12, atol=1e-12)
    for p, v in skip.y_rows.items():
        f = int(full.groups.perm[p]) if p < T * k else None
        if f is not None and mask[full.ids[f // k, f % k]]:
            assert not v.any()
        else:
            assert np.array_equal(v, full.y_rows[p])

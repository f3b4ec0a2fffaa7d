"""Pins of the hot/cold swap policy in the oracle (CPU only).

[Strata] "哪些专家能长期留在显存？", the passages on heat and candidate pairs and on
swaps: heat accumulates routing counts; inside one layer hot experts outside
the cache pair with cold ones inside; a pair is a candidate when the heat gap
reaches the threshold (default 1.5; the page's example: 10 against 8, gap 2);
candidates go by gap, at most 96 a round; then every heat is multiplied by 0.7
and routing keeps adding to it."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _state(heats, resident):
    """heat [L][E] and a slot table [L][E+1] (slot numbers arbitrary, shared resident)."""
    heat = np.array(heats, np.float32)
    L, E = heat.shape
    table = np.full((L, E + 1), -1, np.int32)
    n = 0
    for l in range(L):
        for e in range(E):
            if resident[l][e]:
                table[l, e] = n
                n += 1
        table[l, E] = n
        n += 1
    return heat, table


def test_page_example_gap_two_is_a_candidate():
    # layer 0: outside A (expert 0) heat 10, inside B (expert 1) heat 8 -> gap 2
    # layer 1: outside 9.4, inside 8 -> gap 1.4, below the threshold
    heat, table = _state([[10, 8], [9.4, 8]], [[False, True], [False, True]])
    assert O.swap_plan(heat, table) == [(0, 0, 1)]


@pytest.mark.parametrize("gap,taken", [(1.5, True), (1.25, False)])
def test_threshold_is_inclusive(gap, taken):
    heat, table = _state([[2 + gap, 2]], [[False, True]])
    assert (O.swap_plan(heat, table) == [(0, 0, 1)]) == taken


def test_pairs_hottest_outside_with_coldest_inside_and_stop():
    # outside experts 0, 1, 2 with heat 10, 9, 2; inside 3, 4, 5 with heat 1, 3, 8:
    # pairs (0, 3) gap 9, (1, 4) gap 6, then (2, 5) gap -6 stops the layer
    heat, table = _state([[10, 9, 2, 1, 3, 8]], [[False, False, False, True, True, True]])
    assert O.swap_plan(heat, table) == [(0, 0, 3), (0, 1, 4)]


def test_at_most_max_swaps_by_largest_gap():
    L, E = 25, 8   # 4 candidates per layer, gaps differ by layer: 100 candidates
    heat = np.zeros((L, E), np.float32)
    resident = [[e >= 4 for e in range(E)] for _ in range(L)]
    for l in range(L):
        heat[l, :4] = 100 + l
    heat, table = _state(heat, resident)
    plan = O.swap_plan(heat, table)
    assert len(plan) == 96
    assert {l for l, _, _ in plan} == set(range(1, L))       # layer 0 has the smallest gaps
    assert [l for l, _, _ in plan[:4]] == [24] * 4            # largest gap first


def test_equal_gaps_go_by_layer():
    heat, table = _state([[5, 1], [5, 1]], [[False, True], [False, True]])
    assert O.swap_plan(heat, table) == [(0, 0, 1), (1, 0, 1)]


def test_decay_then_accumulate():
    heat = np.zeros((1, 4), np.float32)
    O.heat_add(heat, 0, np.array([[0, 1], [0, 2], [7, -1]]))   # ids outside [0, E) do not count
    assert list(heat[0]) == [2, 1, 1, 0]
    O.heat_decay(heat)
    O.heat_add(heat, 0, np.array([[0, 3]]))
    np.testing.assert_array_equal(heat[0], np.float32([2 * np.float32(0.7) + 1, np.float32(0.7), np.float32(0.7), 1]))


def test_shared_expert_never_swaps():
    heat, table = _state([[9, 1]], [[False, True]])
    table[0, 2] = -1                          # the shared expert not resident: still no swap for it
    assert O.swap_plan(heat, table) == [(0, 0, 1)]

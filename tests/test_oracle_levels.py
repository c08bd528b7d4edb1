"""Pins of the oracle's frequency-weighted retention (DynamicInfer, key design 2, the
hierarchical neuron cache, importance a + lambda f; slot rule of NeuroPrefetcher section 3.4).

Expected values come from:
  * a hand-worked example with capacity pressure (tests/golden/levels_example.json);
  * closed forms: with room for everything nothing leaves (the resident set is the union of all
    active sets so far); with one level the lowest IDs stay; with no room (|S| = K) the
    resident set is exactly S, so the deltas equal those of the exact rule;
  * a characterisation of the rule checked exhaustively on three-token sequences over 4
    neurons and on long random sequences: S is resident, only resident neurons stay, the kept
    ones are a prefix of the candidates ordered by (level descending, ID ascending), as many as
    fit; together with the slot-machinery invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def resident(ol):
    return set(np.nonzero(ol.slot_map >= 0)[0].tolist())


def test_golden_levels_example():
    g = json.load(open(os.path.join(GOLDEN, "levels_example.json")))
    ol = O.OracleLayer(g["M"], g["K"], 1, 1, keep_buffer=False, levels=np.array(g["levels"]),
                       n_levels=g["n_levels"])
    for st in g["steps"]:
        res = ol.step(np.array(st["S"], dtype=np.int32))
        assert res.d_in.tolist() == st["d_in"], st["note"]
        assert res.slot_in.tolist() == st["slot_in"], st["note"]
        assert res.d_out.tolist() == st["d_out"], st["note"]
        assert sorted(resident(ol)) == st["resident"], st["note"]


def random_sets(rng, M, T, lo, hi):
    return [np.sort(rng.choice(M, int(rng.integers(lo, hi)), replace=False)).astype(np.int32) for _ in range(T)]


def test_no_pressure_keeps_everything():
    rng = np.random.default_rng(1)
    M = 50
    levels = rng.integers(0, 4, M)
    ol = O.OracleLayer(M, M, 1, 1, keep_buffer=False, levels=levels, n_levels=4)
    seen = set()
    for S in random_sets(rng, M, 30, 0, 15):
        res = ol.step(S)
        assert set(res.d_in.tolist()) == set(S.tolist()) - seen and res.d_out.size == 0
        seen |= set(S.tolist())
        assert resident(ol) == seen


def test_one_level_keeps_the_lowest_ids():
    rng = np.random.default_rng(2)
    M, K = 60, 20
    ol = O.OracleLayer(M, K, 1, 1, keep_buffer=False, levels=np.zeros(M), n_levels=1)
    for S in random_sets(rng, M, 40, 3, 15):
        prev = resident(ol)
        ol.step(S)
        cands = sorted(prev - set(S.tolist()))
        assert resident(ol) == set(S.tolist()) | set(cands[: K - S.size])


def test_no_room_is_the_exact_rule():
    rng = np.random.default_rng(3)
    M, K = 40, 12
    levels = rng.integers(0, 8, M)
    ex = O.OracleLayer(M, K, 1, 1, keep_buffer=False)
    lv = O.OracleLayer(M, K, 1, 1, keep_buffer=False, levels=levels, n_levels=8)
    for _ in range(30):
        S = np.sort(rng.choice(M, K, replace=False)).astype(np.int32)  # |S| = K: no room
        a, b = ex.step(S), lv.step(S)
        assert a.d_in.tolist() == b.d_in.tolist() and a.slot_in.tolist() == b.slot_in.tolist()
        assert a.d_out.tolist() == b.d_out.tolist()
        assert np.array_equal(ex.slot_map, lv.slot_map) and np.array_equal(ex.owner, lv.owner)


def check_rule(prev_res, levels, K, S, now_res):
    S = set(S)
    assert S <= now_res and len(now_res) <= K
    kept = now_res - S
    cands = sorted(prev_res - S, key=lambda i: (-int(levels[i]), i))
    assert kept == set(cands[:len(kept)])
    assert len(kept) == min(len(cands), K - len(S))


def check_slots(ol, res, prev_map):
    occ = ol.owner[ol.owner >= 0]
    assert len(set(occ.tolist())) == occ.size
    for n in range(ol.M):
        s = ol.slot_map[n]
        if s >= 0:
            assert ol.owner[s] == n
    for n in res.d_out:
        assert ol.slot_map[n] == -1
    for n in set(np.nonzero(prev_map >= 0)[0].tolist()) - set(res.d_out.tolist()):
        assert ol.slot_map[n] == prev_map[n]
    assert res.slot_in.tolist() == sorted(res.slot_in.tolist())


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("levels", [(0, 1, 2, 3), (1, 0, 1, 0), (2, 2, 0, 1)])
def test_exhaustive_three_token_sequences(K, levels):
    M = 4
    subsets = [s for r in range(0, K + 1) for s in itertools.combinations(range(M), r)]
    for seq in itertools.product(subsets, repeat=3):
        ol = O.OracleLayer(M, K, 1, 1, keep_buffer=False, levels=np.array(levels), n_levels=4)
        for S in seq:
            prev = resident(ol)
            prev_map = ol.slot_map.copy()
            res = ol.step(np.array(S, dtype=np.int32))
            check_rule(prev, levels, K, S, resident(ol))
            check_slots(ol, res, prev_map)


@pytest.mark.parametrize("n_levels", [2, 5, 16])
def test_long_random_sequences_with_pressure(n_levels):
    rng = np.random.default_rng(20 + n_levels)
    M, K = 300, 90
    levels = rng.integers(0, n_levels, M)
    ol = O.OracleLayer(M, K, 1, 1, keep_buffer=False, levels=levels, n_levels=n_levels)
    base = rng.choice(M, 70, replace=False)
    for t in range(120):
        keep = rng.random(base.size) < 0.8
        S = np.unique(np.concatenate([base[keep], rng.choice(M, 15, replace=False)]))[:K].astype(np.int32)
        prev = resident(ol)
        prev_map = ol.slot_map.copy()
        res = ol.step(S)
        check_rule(prev, levels, K, S.tolist(), resident(ol))
        check_slots(ol, res, prev_map)


def test_levels_refuse_over_capacity_and_keep_state():
    ol = O.OracleLayer(10, 3, 1, 1, keep_buffer=False, levels=np.arange(10) % 3, n_levels=3)
    ol.step(np.array([0, 1], dtype=np.int32))
    before = (ol.slot_map.copy(), ol.owner.copy())
    with pytest.raises(O.CapacityError):
        ol.step(np.array([2, 3, 4, 5], dtype=np.int32))
    assert np.array_equal(ol.slot_map, before[0]) and np.array_equal(ol.owner, before[1])


def test_level_out_of_range_is_rejected():
    ol = O.OracleLayer(4, 3, 1, 1, keep_buffer=False, levels=np.array([0, 1, 3, 0]), n_levels=3)
    with pytest.raises(ValueError):
        ol.step(np.array([0], dtype=np.int32))

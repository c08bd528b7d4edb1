"""Pins of the oracle's residency window (LLM in a flash, section 3.1 "Windowing"; slot rule of
NeuroPrefetcher section 3.4).

Expected values come from:
  * a hand-worked example with capacity pressure (tests/golden/window_example.json);
  * the closed form without capacity pressure: the resident set is the union of the last k
    active sets;
  * a characterisation that fixes the retention rule with capacity pressure: S_t is resident,
    only resident neurons of the last k - 1 tokens are kept, more recent ones before older ones,
    lower IDs before higher ones within one token, and as many as fit;
  * exhaustive three-token sequences over 4 neurons, and long random sequences, checked against
    that characterisation and the slot-machinery invariants.
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


def test_golden_window_example():
    g = json.load(open(os.path.join(GOLDEN, "window_example.json")))
    ol = O.OracleLayer(g["M"], g["K"], 1, 1, keep_buffer=False, window=g["k"])
    for st in g["steps"]:
        res = ol.step(np.array(st["S"], dtype=np.int32))
        assert res.d_in.tolist() == st["d_in"], st["note"]
        assert res.slot_in.tolist() == st["slot_in"], st["note"]
        assert res.d_out.tolist() == st["d_out"], st["note"]
        assert sorted(resident(ol)) == st["resident"], st["note"]


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_no_capacity_pressure_is_the_union_of_the_last_k_sets(k):
    rng = np.random.default_rng(k)
    M = 60
    ol = O.OracleLayer(M, M, 1, 1, keep_buffer=False, window=k)
    hist = []
    for t in range(40):
        S = np.sort(rng.choice(M, int(rng.integers(0, 20)), replace=False)).astype(np.int32)
        prev = set().union(*hist[-k:]) if hist else set()
        res = ol.step(S)
        hist.append(set(S.tolist()))
        window = set().union(*hist[-k:])
        assert resident(ol) == window
        assert set(res.d_in.tolist()) == set(S.tolist()) - prev
        assert set(res.d_out.tolist()) == prev - window


def test_larger_windows_never_load_more_without_pressure():
    rng = np.random.default_rng(3)
    M, T = 80, 60
    seq = [np.sort(rng.choice(M, int(rng.integers(5, 30)), replace=False)).astype(np.int32) for _ in range(T)]
    loads = []
    for k in (1, 2, 4, 8):
        ol = O.OracleLayer(M, M, 1, 1, keep_buffer=False, window=k)
        loads.append(sum(ol.step(S).d_in.size for S in seq))
    assert loads == sorted(loads, reverse=True) and loads[0] > loads[-1]


def check_rule(prev_res, last, t, k, K, S, now_res):
    """The characterisation of one window step (last: last active token before t)."""
    S = set(S)
    assert S <= now_res and len(now_res) <= K
    kept = now_res - S
    cands = [i for i in prev_res - S if 1 <= t - last[i] < k]
    assert kept <= set(cands)
    order = sorted(cands, key=lambda i: (t - last[i], i))          # priority order
    assert kept == set(order[:len(kept)])                            # a prefix of it ...
    assert len(kept) == min(len(cands), K - len(S))                  # ... as long as it fits


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
        assert ol.slot_map[n] == prev_map[n]                         # survivors keep their slot
    assert res.slot_in.tolist() == sorted(res.slot_in.tolist())


@pytest.mark.parametrize("K,k", [(2, 2), (3, 2), (3, 3), (4, 3), (4, 2)])
def test_exhaustive_three_token_sequences(K, k):
    M = 4
    subsets = [s for r in range(0, K + 1) for s in itertools.combinations(range(M), r)]
    for seq in itertools.product(subsets, repeat=3):
        ol = O.OracleLayer(M, K, 1, 1, keep_buffer=False, window=k)
        last = {i: -10 for i in range(M)}
        for t, S in enumerate(seq):
            prev = resident(ol)
            prev_map = ol.slot_map.copy()
            res = ol.step(np.array(S, dtype=np.int32))
            check_rule(prev, last, t, k, K, S, resident(ol))
            check_slots(ol, res, prev_map)
            for i in S:
                last[i] = t


@pytest.mark.parametrize("k", [2, 4, 16])
def test_long_random_sequences_with_pressure(k):
    rng = np.random.default_rng(10 + k)
    M, K = 300, 90
    ol = O.OracleLayer(M, K, 1, 1, keep_buffer=False, window=k)
    last = {i: -100 for i in range(M)}
    base = rng.choice(M, 70, replace=False)
    for t in range(120):
        keep = rng.random(base.size) < 0.8
        S = np.unique(np.concatenate([base[keep], rng.choice(M, 15, replace=False)]))[:K].astype(np.int32)
        prev = resident(ol)
        prev_map = ol.slot_map.copy()
        res = ol.step(S)
        check_rule(prev, last, t, k, K, S.tolist(), resident(ol))
        check_slots(ol, res, prev_map)
        assert ol.active_slots(S).tolist() == sorted(ol.slot_map[S].tolist())
        for i in S.tolist():
            last[i] = t


def test_window_refuses_over_capacity_and_keeps_state():
    ol = O.OracleLayer(10, 3, 1, 1, keep_buffer=False, window=4)
    ol.step(np.array([0, 1], dtype=np.int32))
    before = (ol.slot_map.copy(), ol.owner.copy(), ol.last_t.copy(), ol.t)
    with pytest.raises(O.CapacityError):
        ol.step(np.array([2, 3, 4, 5], dtype=np.int32))
    assert np.array_equal(ol.slot_map, before[0]) and np.array_equal(ol.owner, before[1])
    assert np.array_equal(ol.last_t, before[2]) and ol.t == before[3]

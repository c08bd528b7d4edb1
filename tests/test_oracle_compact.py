"""Pins of the oracle's compacted buffer (LLM in a flash, section 3.3: the occupied rows form
a prefix, a removed row is replaced by a row from the end of the region, incoming rows are
appended; the set difference of NeuroPrefetcher section 3.4 decides who leaves and comes).

Expected values come from:
  * a hand-worked example (tests/golden/compact_example.json);
  * a closed form of the moves: with n_keep = |R| - |D_out|, the holes (positions below n_keep
    whose neuron leaves, ascending) are paired with the rows that stay at positions n_keep and
    above (descending), and the incoming neurons take positions n_keep, n_keep + 1, ...;
  * the exact rule's set difference (the slot oracle gives the same D_in and D_out, and the
    buffer holds exactly S at positions 0 .. |S|-1);
  * the buffer contents: after copying, the row at each active neuron's position is that
    neuron's bundle;
checked exhaustively on short sequences over 5 neurons and on long random sequences.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_compact_example():
    g = json.load(open(os.path.join(GOLDEN, "compact_example.json")))
    ol = O.OracleLayer(g["M"], g["K"], 1, 1, keep_buffer=False, layout="compact")
    for st in g["steps"]:
        res = ol.step(np.array(st["S"], dtype=np.int32))
        for key, got in (("d_in", res.d_in), ("pos_in", res.slot_in), ("d_out", res.d_out),
                         ("mv_src", res.mv_src), ("mv_dst", res.mv_dst), ("owner", ol.owner)):
            assert got.tolist() == st[key], (key, st["note"])


def closed_form(owner, n_occ, S):
    S = set(S)
    R = [int(owner[p]) for p in range(n_occ)]
    d_out = sorted(set(R) - S)
    d_in = sorted(S - set(R))
    n_keep = n_occ - len(d_out)
    holes = [p for p in range(n_keep) if R[p] not in S]
    movers = [p for p in range(n_occ - 1, n_keep - 1, -1) if R[p] in S]
    assert len(holes) == len(movers)
    return d_in, d_out, movers, holes, list(range(n_keep, n_keep + len(d_in)))


def check_step(ol, prev_owner, prev_n, S, res, ex, store=None):
    d_in, d_out, movers, holes, pos_in = closed_form(prev_owner, prev_n, S)
    assert res.d_in.tolist() == d_in and res.d_out.tolist() == d_out
    assert res.mv_src.tolist() == movers and res.mv_dst.tolist() == holes
    assert res.slot_in.tolist() == pos_in
    n = len(S)
    assert ol.n_occ == n and sorted(ol.owner[:n].tolist()) == sorted(S)
    assert (ol.owner[n:] == -1).all()
    for p in range(n):
        assert ol.slot_map[ol.owner[p]] == p
    assert (ol.slot_map >= 0).sum() == n
    moved = set(res.mv_dst.tolist()) | set(pos_in)
    for p in range(n):                      # rows neither moved nor appended stay put
        if p not in moved:
            assert ol.owner[p] == prev_owner[p]
    # same set difference as the slot layout
    er = ex.step(np.array(sorted(S), dtype=np.int32))
    assert er.d_in.tolist() == d_in and er.d_out.tolist() == d_out
    if store is not None:
        ol.copy_bundles(store, res)
        for p in range(n):
            assert np.array_equal(ol.buf[p], store[ol.owner[p]])


@pytest.mark.parametrize("K", [2, 3, 5])
def test_exhaustive_short_sequences(K):
    M = 5
    subsets = [s for r in range(0, K + 1) for s in itertools.combinations(range(M), r)]
    store = np.arange(M * 2, dtype=np.uint16).reshape(M, 1, 2) + 1
    for seq in itertools.product(subsets, repeat=3):
        ol = O.OracleLayer(M, K, 1, 2, layout="compact")
        ex = O.OracleLayer(M, K, 1, 2, keep_buffer=False)
        for S in seq:
            prev_owner, prev_n = ol.owner.copy(), ol.n_occ
            res = ol.step(np.array(S, dtype=np.int32))
            check_step(ol, prev_owner, prev_n, list(S), res, ex, store)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_long_random_sequences(seed):
    rng = np.random.default_rng(40 + seed)
    M, K, R, d = 400, 150, 2, 4
    store = rng.integers(0, 65535, size=(M, R, d), dtype=np.uint16)
    ol = O.OracleLayer(M, K, R, d, layout="compact")
    ex = O.OracleLayer(M, K, R, d, keep_buffer=False)
    cur = rng.choice(M, 100, replace=False)
    for t in range(150):
        keep = cur[rng.random(cur.size) < 0.8]
        add = rng.choice(M, int(rng.integers(0, 50)), replace=False)
        cur = np.unique(np.concatenate([keep, add]))[:K]
        S = np.sort(cur).astype(np.int32)
        prev_owner, prev_n = ol.owner.copy(), ol.n_occ
        res = ol.step(S)
        check_step(ol, prev_owner, prev_n, S.tolist(), res, ex, store)
        assert res.mv_src.size <= res.d_out.size


def test_compact_refuses_over_capacity_and_keeps_state():
    ol = O.OracleLayer(10, 3, 1, 1, keep_buffer=False, layout="compact")
    ol.step(np.array([0, 1], dtype=np.int32))
    before = (ol.slot_map.copy(), ol.owner.copy(), ol.n_occ)
    with pytest.raises(O.CapacityError):
        ol.step(np.array([2, 3, 4, 5], dtype=np.int32))
    assert np.array_equal(ol.slot_map, before[0]) and np.array_equal(ol.owner, before[1])
    assert ol.n_occ == before[2]

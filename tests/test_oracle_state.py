"""Pins of the oracle's set machinery (active set, delta, slot assignment).

What fixes the expected values here, none of which comes from the HIP path:
  * the worked example of the DynamicInfer notes page, run through the delta
    rule of NeuroPrefetcher section 3.4 (tests/golden/dynamicinfer_example.json);
  * closed forms: cold start gives slots 0..n-1; S == R gives empty deltas;
    S and R disjoint gives full turnover;
  * invariants that must hold after every step (section 3.4: the buffer holds
    exactly the active set, the slot map is -1 for non-resident neurons,
    persisting rows keep their slot because compaction is avoided);
  * mask combination against NumPy's bitwise routines;
  * exhaustive small cases checked against those invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
from workload.gen import ids_to_words

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_invariants(layer: O.OracleLayer, S, R_prev, prev_slot_map, res: O.StepResult):
    S = set(int(i) for i in S)
    R_prev = set(int(i) for i in R_prev)
    # I1, I2: delta sizes are the set-difference sizes, lists ascending and exact
    assert res.d_in.tolist() == sorted(S - R_prev)
    assert res.d_out.tolist() == sorted(R_prev - S)
    # I3: the occupied slots hold exactly S
    held = {int(n) for n in layer.owner if n != -1}
    assert held == S
    # I4: slot map and owner table are inverse maps; -1 elsewhere
    for n in range(layer.M):
        s = int(layer.slot_map[n])
        if n in S:
            assert s >= 0 and layer.owner[s] == n
        else:
            assert s == -1
    # I5: persisting neurons keep their slot
    for n in S & R_prev:
        assert layer.slot_map[n] == prev_slot_map[n]
    # I7: free slot count
    assert int((layer.owner == -1).sum()) == layer.K - len(S)
    # deterministic assignment: slot_in is the |D_in| smallest slots free after the release
    free_after_release = sorted(set(range(layer.K)) - {int(prev_slot_map[n]) for n in S & R_prev})
    assert res.slot_in.tolist() == free_after_release[: len(res.d_in)]


def test_golden_dynamicinfer_example():
    g = json.load(open(os.path.join(GOLDEN, "dynamicinfer_example.json")))
    layer = O.OracleLayer(g["M"], g["K"], 1, 8, keep_buffer=False)
    for st in g["steps"]:
        res = layer.step(np.array(st["active"]))
        assert res.d_in.tolist() == st["d_in"]
        assert res.slot_in.tolist() == st["slot_in"]
        assert res.d_out.tolist() == st["d_out"]
        assert layer.owner.tolist() == st["owner"]
        assert layer.slot_map.tolist() == st["slot_map"]


def test_cold_start_fills_slots_in_order():
    rng = np.random.default_rng(1)
    M, K = 500, 120
    S = np.sort(rng.choice(M, size=97, replace=False))
    layer = O.OracleLayer(M, K, 3, 8, keep_buffer=False)
    res = layer.step(S)
    assert res.d_in.tolist() == S.tolist()
    assert res.slot_in.tolist() == list(range(97))
    assert res.d_out.size == 0
    assert layer.occupied_slots().tolist() == list(range(97))


def test_same_set_gives_empty_delta():
    M, K = 300, 64
    S = np.arange(5, 300, 7)
    layer = O.OracleLayer(M, K, 3, 8, keep_buffer=False)
    layer.step(S)
    before = layer.slot_map.copy()
    res = layer.step(S)
    assert res.d_in.size == 0 and res.d_out.size == 0
    assert (layer.slot_map == before).all()


def test_full_turnover_reuses_slots_ascending():
    M, K = 200, 50
    A = np.arange(0, 100, 2)     # 50 neurons: exactly K
    B = np.arange(1, 101, 2)     # disjoint, also 50
    layer = O.OracleLayer(M, K, 3, 8, keep_buffer=False)
    layer.step(A)
    res = layer.step(B)
    assert res.d_out.tolist() == A.tolist()
    assert res.d_in.tolist() == B.tolist()
    assert res.slot_in.tolist() == list(range(50))


def test_capacity_exact_and_overflow_leaves_state_unchanged():
    M, K = 128, 16
    layer = O.OracleLayer(M, K, 3, 8, keep_buffer=False)
    layer.step(np.arange(16))                       # |S| == K is fine
    sm, ow = layer.slot_map.copy(), layer.owner.copy()
    with pytest.raises(O.CapacityError):
        layer.step(np.arange(100, 117))             # 17 > K
    assert (layer.slot_map == sm).all() and (layer.owner == ow).all()
    res = layer.step(np.array([], dtype=np.int32))  # empty set releases everything
    assert res.d_out.tolist() == list(range(16)) and res.d_in.size == 0
    assert (layer.owner == -1).all() and (layer.slot_map == -1).all()


def test_copy_bundles_places_rows_and_keeps_stale_rows():
    rng = np.random.default_rng(7)
    M, K, R, d = 40, 8, 3, 16
    store = rng.integers(0, 2**16, size=(M, R, d), dtype=np.uint16)
    layer = O.OracleLayer(M, K, R, d)
    seq = [[1, 2, 3, 4, 5], [2, 3, 9, 10], [30, 31, 32, 33, 34, 35, 36, 37]]
    written = {}
    for S in seq:
        res = layer.step(np.array(S))
        layer.copy_bundles(store, res)
        for n, s in zip(res.d_in, res.slot_in):
            written[int(s)] = int(n)
        for s in range(K):
            if s in written:
                assert (layer.buf[s] == store[written[s]]).all()   # I6 and stale rows
            else:
                assert (layer.buf[s] == 0).all()


def _np_combine(a, b, M, mode):
    if mode == O.UNION:
        w = np.bitwise_or(a, b)
    elif mode == O.INTERSECT:
        w = np.bitwise_and(a, b)
    else:
        w = a
    bits = np.unpackbits(w.astype("<u8").view(np.uint8), bitorder="little")[:M]
    return np.nonzero(bits)[0]


@pytest.mark.parametrize("M", [1, 63, 64, 65, 200, 1024])
@pytest.mark.parametrize("mode", [O.UNION, O.INTERSECT, O.SINGLE])
def test_active_set_matches_numpy_bit_ops(M, mode):
    rng = np.random.default_rng(M * 10 + mode)
    for _ in range(5):
        a = ids_to_words(np.nonzero(rng.random(M) < 0.3)[0], M)
        b = ids_to_words(np.nonzero(rng.random(M) < 0.3)[0], M)
        got = O.active_set(a, b, M, mode)
        assert got.tolist() == _np_combine(a, b, M, mode).tolist()
        if mode == O.UNION:   # inclusion-exclusion closed form
            ia = O.active_set(a, a, M, O.SINGLE)
            ib = O.active_set(b, b, M, O.SINGLE)
            ii = O.active_set(a, b, M, O.INTERSECT)
            assert got.size == ia.size + ib.size - ii.size


def test_active_set_hand_masks():
    # neuron 0, 5 and 70 in gate; 5, 64 and 127 in up
    g = np.array([(1 << 0) | (1 << 5), 1 << 6], dtype=np.uint64)
    u = np.array([1 << 5, (1 << 0) | (1 << 63)], dtype=np.uint64)
    assert O.active_set(g, u, 128, O.UNION).tolist() == [0, 5, 64, 70, 127]
    assert O.active_set(g, u, 128, O.INTERSECT).tolist() == [5]
    assert O.active_set(g, u, 128, O.SINGLE).tolist() == [0, 5, 70]


@pytest.mark.parametrize("K", [2, 3, 5])
def test_exhaustive_three_step_sequences(K):
    """Every sequence of 3 subsets of 5 neurons: invariants after every step, refusals when |S| > K."""
    M = 5
    subsets = [np.array([i for i in range(M) if (mask >> i) & 1], dtype=np.int32) for mask in range(1 << M)]
    for seq in itertools.product(range(len(subsets)), repeat=3):
        layer = O.OracleLayer(M, K, 1, 8, keep_buffer=False)
        R = np.array([], dtype=np.int32)
        for idx in seq:
            S = subsets[idx]
            prev = layer.slot_map.copy()
            if S.size > K:
                ow = layer.owner.copy()
                with pytest.raises(O.CapacityError):
                    layer.step(S)
                assert (layer.slot_map == prev).all() and (layer.owner == ow).all()
                continue
            res = layer.step(S)
            check_invariants(layer, S, R, prev, res)
            R = S


def test_random_long_sequences_keep_invariants():
    rng = np.random.default_rng(11)
    M, K = 700, 160
    layer = O.OracleLayer(M, K, 1, 8, keep_buffer=False)
    R = np.array([], dtype=np.int32)
    for t in range(60):
        n = int(rng.integers(0, K + 1))
        keep = rng.choice(R, size=min(R.size, int(n * rng.uniform(0, 1))), replace=False) if R.size else np.array([], dtype=np.int64)
        pool = np.setdiff1d(np.arange(M), keep)
        S = np.sort(np.concatenate([keep, rng.choice(pool, size=n - keep.size, replace=False)])).astype(np.int32)
        prev = layer.slot_map.copy()
        res = layer.step(S)
        check_invariants(layer, S, R, prev, res)
        R = S

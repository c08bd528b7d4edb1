"""Pins of the oracle's sparse FFN (fp64).

Expected values come from:
  * hand-worked examples (tests/golden/tiny_ffn_hand.json);
  * the dense FFN with inactive neurons masked, evaluated with NumPy's matrix
    product in fp64 (NeuroPrefetcher section 3.4: only active neurons
    contribute, each through row i of gate, up and down^T);
  * exact integer arithmetic on dyadic inputs;
  * closed forms for |S| = 0 and |S| = 1;
  * invariance under a consistent relabelling of neurons (LLM in a flash,
    section 3.3; NeuroPrefetcher section 3.4: row order does not matter).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from workload.gen import CONFIGS, Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def to_bf16_bits(a):
    """Exact fp32 -> bf16 bits (the values used here are exact in bf16)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32)
    assert (u & 0xFFFF == 0).all(), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_masked(store_bits, R, x, active):
    """fp64 dense FFN over ALL neurons with a 0/1 mask, via NumPy matmul."""
    W = bf16_to_f64(store_bits)          # [M][R][d]
    x64 = np.asarray(x, dtype=np.float64)
    m = np.zeros(W.shape[0])
    m[np.asarray(active, dtype=np.int64)] = 1.0
    if R == 3:
        g = W[:, 0, :] @ x64
        u = W[:, 1, :] @ x64
        h = m * np.maximum(g, 0.0) * u
    else:
        u = W[:, 0, :] @ x64
        h = m * np.maximum(u, 0.0)
    return W[:, R - 1, :].T @ h


@pytest.mark.parametrize("kind", ["gated", "nongated"])
def test_golden_hand_examples(kind):
    g = json.load(open(os.path.join(GOLDEN, "tiny_ffn_hand.json")))
    case = g[kind]
    store = to_bf16_bits(np.array(case["bundles"], dtype=np.float32))
    R = store.shape[1]
    y = O.sparse_ffn(store, R, 4, np.array(case["active"]), np.array(g["x"], dtype=np.float32))
    assert y.tolist() == case["y"]


@pytest.mark.parametrize("seed", range(4))
def test_sparse_equals_dense_masked_config1_shape(seed):
    c = CONFIGS[1]
    wl = Workload(c)
    store = wl.store(0)
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, c.K + 1))
    S = np.sort(rng.choice(c.M, size=n, replace=False))
    x = wl.x(seed, 0)
    y = O.sparse_ffn(store, c.R, c.d, S, x)
    ref = dense_masked(store, c.R, x, S)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_full_active_set_is_the_dense_ffn():
    rng = np.random.default_rng(3)
    M, d = 96, 48
    Wg = rng.standard_normal((M, d)).astype(np.float32) * 0.1
    Wu = rng.standard_normal((M, d)).astype(np.float32) * 0.1
    Wd = rng.standard_normal((d, M)).astype(np.float32) * 0.1   # down projection, d x M
    # round to bf16 once so both sides see the same weights
    Wg, Wu, Wd = [bf16_to_f64(to_bf16_bits_rne(w)) for w in (Wg, Wu, Wd)]
    x = rng.standard_normal(d).astype(np.float32)
    store = np.stack([to_bf16_bits(Wg.astype(np.float32)), to_bf16_bits(Wu.astype(np.float32)),
                      to_bf16_bits(Wd.T.astype(np.float32))], axis=1)
    y = O.sparse_ffn(np.ascontiguousarray(store), 3, d, np.arange(M), x)
    x64 = x.astype(np.float64)
    ref = Wd @ (np.maximum(Wg @ x64, 0.0) * (Wu @ x64))        # textbook gated ReLU FFN
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def to_bf16_bits_rne(a):
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_empty_and_single_neuron_closed_forms():
    c = CONFIGS[1]
    wl = Workload(c)
    store = wl.store(0)
    x = wl.x(0, 0)
    y0 = O.sparse_ffn(store, c.R, c.d, np.array([], dtype=np.int32), x)
    assert (y0 == 0.0).all()
    x64 = x.astype(np.float64)
    for n in (0, 17, c.M - 1):
        W = bf16_to_f64(store[n])
        g, u = W[0] @ x64, W[1] @ x64
        h = max(g, 0.0) * u
        y1 = O.sparse_ffn(store, c.R, c.d, np.array([n]), x)
        assert np.abs(y1 - h * W[2]).max() <= 1e-14 * max(1e-30, np.abs(h * W[2]).max())


@pytest.mark.parametrize("R", [3, 2])
def test_exact_dyadic_inputs_match_integer_arithmetic(R):
    """Weights k/64 (|k| <= 8), x = j/8 (|j| <= 8): every value is exact; compare bit-for-bit."""
    rng = np.random.default_rng(5 + R)
    M, d = 40, 256
    wk = rng.integers(-8, 9, size=(M, R, d))
    xj = rng.integers(-8, 9, size=d)
    store = to_bf16_bits((wk / 64.0).astype(np.float32))
    x = (xj / 8.0).astype(np.float32)
    S = np.sort(rng.choice(M, size=25, replace=False))
    y = O.sparse_ffn(store, R, d, S, x)
    exact = [Fraction(0)] * d
    for n in S:
        if R == 3:
            g = Fraction(int(np.dot(wk[n, 0], xj)), 64 * 8)
            u = Fraction(int(np.dot(wk[n, 1], xj)), 64 * 8)
            h = max(g, Fraction(0)) * u
        else:
            u = Fraction(int(np.dot(wk[n, 0], xj)), 64 * 8)
            h = max(u, Fraction(0))
        for j in range(d):
            exact[j] += h * Fraction(int(wk[n, R - 1, j]), 64)
    assert [Fraction(v) for v in y.tolist()] == exact


def test_nongated_equals_dense_masked():
    rng = np.random.default_rng(9)
    M, d = 300, 128
    store = to_bf16_bits_rne(rng.standard_normal((M, 2, d)).astype(np.float32) * 0.05)
    x = rng.standard_normal(d).astype(np.float32)
    S = np.sort(rng.choice(M, size=77, replace=False))
    y = O.sparse_ffn(store, 2, d, S, x)
    ref = dense_masked(store, 2, x, S)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_consistent_relabelling_preserves_output():
    c = CONFIGS[1]
    wl = Workload(c)
    store = wl.store(0)
    rng = np.random.default_rng(21)
    S = np.sort(rng.choice(c.M, size=300, replace=False))
    x = wl.x(2, 0)
    y = O.sparse_ffn(store, c.R, c.d, S, x)
    perm = rng.permutation(c.M)              # neuron n moves to position perm[n]
    permuted = np.empty_like(store)
    permuted[perm] = store
    y2 = O.sparse_ffn(permuted, c.R, c.d, np.sort(perm[S]), x)
    assert np.abs(y - y2).max() <= 1e-12 * np.abs(y).max()


def test_relu_zero_boundary():
    # gate . x == 0 exactly: relu(0) = 0, so the neuron contributes nothing
    store = to_bf16_bits(np.array([[[1.0, -1.0], [3.0, 3.0], [1.0, 1.0]]], dtype=np.float32))
    y = O.sparse_ffn(store, 3, 2, np.array([0]), np.array([1.0, 1.0], dtype=np.float32))
    assert y.tolist() == [0.0, 0.0]


# ---- SiLU (the gate of the paper's SwiGLU MLPs, NeuroPrefetcher section 3.4) ----
# silu(g) = g * sigmoid(g). The pins use facts of the logistic function that do not restate
# the formula: sigmoid(ln a) = a / (1 + a) for a > 0, sigmoid(-g) = 1 - sigmoid(g) (so that
# silu(g) - silu(-g) = g), and the limits silu(g) -> g for large g, -> 0 for very negative g.

def _one_neuron(gate, up, down, R):
    rows = [gate, up, down] if R == 3 else [up, down]
    return to_bf16_bits(np.array([[[r] for r in rows]], dtype=np.float32))


@pytest.mark.parametrize("a", [3.0, 2.0, 0.5, 9.0])
def test_silu_at_log_points(a):
    # gated, d = 1, gate = up = down = 1: y = silu(x) * x with x = fp32(ln a); sigmoid(ln a)
    # = a / (1 + a), and fp32 rounding of ln a moves it by at most 1e-7 relative
    x = np.float32(np.log(a))
    y = O.sparse_ffn(_one_neuron(1.0, 1.0, 1.0, 3), 3, 1, np.array([0]), np.array([x]), "silu")[0]
    want = (a / (1.0 + a)) * float(x) * float(x)
    assert abs(y - want) <= 1e-7 * abs(want)


def test_silu_odd_part_is_identity():
    # non-gated, up = down = 1: y(x) = silu(x); silu(x) - silu(-x) = x exactly in real arithmetic
    rng = np.random.default_rng(5)
    st = _one_neuron(0.0, 1.0, 1.0, 2)
    for x in rng.standard_normal(50).astype(np.float32) * 4:
        yp = O.sparse_ffn(st, 2, 1, np.array([0]), np.array([x]), "silu")[0]
        ym = O.sparse_ffn(st, 2, 1, np.array([0]), np.array([-x]), "silu")[0]
        assert abs((yp - ym) - float(x)) <= 1e-14 * max(1.0, abs(float(x)))
        assert (yp > 0) == (x > 0) or x == 0                  # silu keeps the sign
        assert ym >= -0.2785                                    # its minimum is about -0.2785


def test_silu_limits_and_zero():
    st = _one_neuron(0.0, 1.0, 1.0, 2)
    y = lambda x: O.sparse_ffn(st, 2, 1, np.array([0]), np.array([x], dtype=np.float32), "silu")[0]
    assert y(0.0) == 0.0
    assert abs(y(40.0) - 40.0) <= 40.0 * 1e-15
    assert abs(y(-40.0)) <= 1e-15


def test_silu_gated_equals_dense_masked():
    # the sparse sum over S equals the dense SwiGLU FFN with inactive neurons masked (dense
    # side: NumPy matmul; its activation from the log-point fact sigmoid(g) = e^g / (1 + e^g))
    rng = np.random.default_rng(11)
    M, d = 64, 48
    store = (rng.standard_normal((M, 3, d)).astype(np.float32) * 0.25)
    store = ((store.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # round to bf16 bits
    x = rng.standard_normal(d).astype(np.float32)
    active = np.sort(rng.choice(M, 20, replace=False)).astype(np.int32)
    W = bf16_to_f64(store)
    g = W[:, 0, :] @ x.astype(np.float64)
    u = W[:, 1, :] @ x.astype(np.float64)
    eg = np.exp(g)
    m = np.zeros(M)
    m[active] = 1.0
    want = W[:, 2, :].T @ (m * g * (eg / (1.0 + eg)) * u)
    y = O.sparse_ffn(store, 3, d, active, x, "silu")
    assert np.abs(y - want).max() <= 1e-12 * np.abs(want).max()


def test_unknown_activation_is_refused():
    st = _one_neuron(1.0, 1.0, 1.0, 3)
    with pytest.raises(KeyError):
        O.sparse_ffn(st, 3, 1, np.array([0]), np.array([1.0], dtype=np.float32), "gelu")

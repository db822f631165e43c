"""Pins of the oracle's routed-expert layer (routing, combine, the whole layer),
independent of its own code: a hand-routed example, permutation invariants, and
reductions to the already pinned grouped and dense products."""

import numpy as np
import pytest

import oracle
import synth


def test_route_hand_example():
    # tokens 0..2, top-2: (t0: 2, 0), (t1: 2, 1), (t2: 0, 2) -> expert 0 gets (0,1) (2,0);
    # expert 1 gets (1,1); expert 2 gets (0,0) (1,0) (2,1); expert 3 gets nothing
    ids = np.array([[2, 0], [2, 1], [0, 2]])
    offsets, tok, slot, row = oracle.moe_route(ids, 4)
    assert offsets.tolist() == [0, 2, 3, 6, 6]
    assert tok.tolist() == [0, 2, 1, 0, 1, 2]
    assert slot.tolist() == [1, 0, 1, 0, 0, 1]
    assert row.tolist() == [[3, 0], [4, 2], [1, 5]]
    with pytest.raises(ValueError):
        oracle.moe_route(np.array([[4, 0]]), 4)


def test_route_is_a_sorted_permutation():
    rng = np.random.default_rng(3)
    ids = np.stack([rng.choice(64, 6, replace=False) for _ in range(200)])
    offsets, tok, slot, row = oracle.moe_route(ids, 64)
    p = ids.size
    assert offsets[0] == 0 and offsets[-1] == p and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.diff(offsets), np.bincount(ids.ravel(), minlength=64))
    # every (t, j) appears once, at the row pair_row names, under its expert's range
    assert sorted(row.ravel().tolist()) == list(range(p))
    for t in range(200):
        for j in range(6):
            rr = row[t, j]
            assert tok[rr] == t and slot[rr] == j and offsets[ids[t, j]] <= rr < offsets[ids[t, j] + 1]


def _bank(rng, experts, n, k, group):
    q = np.stack([synth.integer_codes(rng, n, k) for _ in range(experts)])
    s = np.stack([synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3) for _ in range(experts)])
    return np.stack([oracle.pack(q[e]) for e in range(experts)]), s


def test_layer_reduces_to_grouped_and_dense():
    rng = np.random.default_rng(4)
    experts, n, k, t_count, topk = 6, 48, 64, 9, 2
    packed, s = _bank(rng, experts, n, k, 32)
    x = synth.integer_activations(rng, t_count, k)
    ids = np.stack([rng.choice(experts, topk, replace=False) for _ in range(t_count)])
    w = rng.integers(-3, 4, size=(t_count, topk)).astype(np.float32) / 4
    offsets, tok, slot, row = oracle.moe_route(ids, experts)
    y_pairs = oracle.grouped_linear(x[tok], packed, s, offsets, 32)
    # route -> grouped product -> combine is the layer
    assert np.array_equal(oracle.moe_combine(y_pairs, row, w), oracle.moe_layer(x, ids, w, packed, s, 32))
    # one expert for every token, weight 1: the dense product of that expert
    ones = np.ones((t_count, 1), np.float32)
    zero_ids = np.zeros((t_count, 1), np.int64)
    assert np.array_equal(oracle.moe_layer(x, zero_ids, ones, packed, s, 32), oracle.linear(x, packed[0], s[0], 32))
    # linear in the router weights (exact for a power of two)
    assert np.array_equal(oracle.moe_layer(x, ids, 2 * w, packed, s, 32), 2 * oracle.moe_layer(x, ids, w, packed, s, 32))


def test_combine_brute_force():
    rng = np.random.default_rng(5)
    y_pairs = rng.standard_normal((12, 5))
    row = rng.permutation(12).reshape(4, 3)
    w = rng.standard_normal((4, 3)).astype(np.float32)
    out = oracle.moe_combine(y_pairs, row, w)
    for t in range(4):
        for c in range(5):
            want = sum(float(w[t, j]) * y_pairs[row[t, j], c] for j in range(3))
            assert abs(out[t, c] - want) <= 1e-12 * max(1.0, abs(want))


def test_combine_hand_example():
    """Two tokens, two slots, values worked out by hand: the combine pairs slot j's
    router weight with the row that pair_row names for (t, j), not with row j."""
    # grouped rows (e.g. sorted by expert): row r holds the product of one (token, slot) pair
    y_pairs = np.array([[1.0, 10.0],     # row 0: (token 1, slot 0)
                        [2.0, 20.0],     # row 1: (token 0, slot 1)
                        [3.0, 30.0],     # row 2: (token 0, slot 0)
                        [4.0, 40.0]])    # row 3: (token 1, slot 1)
    pair_row = np.array([[2, 1], [0, 3]])
    w = np.array([[0.5, 0.25], [2.0, -1.0]], np.float32)
    out = oracle.moe_combine(y_pairs, pair_row, w)
    # token 0: 0.5 * row 2 + 0.25 * row 1 = (1.5 + 0.5, 15 + 5)
    # token 1: 2 * row 0 - 1 * row 3 = (2 - 4, 20 - 40)
    assert out.tolist() == [[2.0, 20.0], [-2.0, -20.0]]

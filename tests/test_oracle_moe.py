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


def _unit_bank(codes_per_row, k, group, scale):
    """One expert whose weight rows have the given {position: code} maps, all scales `scale`."""
    q = np.zeros((len(codes_per_row), k), np.int8)
    for r, m in enumerate(codes_per_row):
        for pos, c in m.items():
            q[r, pos] = c
    s = np.full((len(codes_per_row), k // group), scale, np.float16)
    return oracle.pack(q)[None], s[None]


def test_moe_ffn_hand_example():
    """One token routed to one expert with router weight 1/2, values worked out by hand.

    x = 32 ones.  Gate/up rows interleave (row 2i gate, 2i + 1 up), scale 1:
    pair 0: gate = 8 codes of 5 -> g = 40, SiLU(40) = 40 in fp64; up = one 3 -> u = 3; h0 = 120
    pair 1: gate = 40 again, up = one -1 -> h1 = -40; pairs 2..31 all zero -> h = 0.
    Down (k = 32 = the 32 pairs): row 0 codes 1 at 0, 2 at 1, scale 1/2 -> (120 - 80) / 2 = 20;
    row 1 code -1 at 0, scale 1/4 -> -30.  out = 1/2 * (20, -30) = (10, -15).
    """
    gate40 = {p: 5 for p in range(8)}
    rows = [gate40, {3: 3}, gate40, {7: -1}] + [{}] * 60
    gu_p, gu_s = _unit_bank(rows, 32, 32, 1.0)
    dn_p0, dn_s0 = _unit_bank([{0: 1, 1: 2}], 32, 32, 0.5)
    dn_p1, dn_s1 = _unit_bank([{0: -1}], 32, 32, 0.25)
    dn_p, dn_s = np.concatenate([dn_p0, dn_p1], axis=1), np.concatenate([dn_s0, dn_s1], axis=1)
    x = np.ones((1, 32), np.float16)
    out = oracle.moe_ffn(x, np.array([[0]]), np.array([[0.5]], np.float32), gu_p, gu_s, dn_p, dn_s, 32)
    assert out.tolist() == [[10.0, -15.0]]
    # gate and up swapped in the bank: SiLU(3) * 40 is not an integer, so the example would fail
    swapped = [rows[1], rows[0], rows[3], rows[2]] + rows[4:]
    gu_q, _ = _unit_bank(swapped, 32, 32, 1.0)
    assert oracle.moe_ffn(x, np.array([[0]]), np.array([[0.5]], np.float32), gu_q, gu_s, dn_p, dn_s,
                          32).tolist() != [[10.0, -15.0]]


def test_grouped_swiglu_is_silu_of_gate_times_up():
    """The grouped SwiGLU product equals SiLU of the grouped product over the gate (even)
    rows times the grouped product over the up (odd) rows, expert by expert."""
    rng = np.random.default_rng(8)
    experts, n, k = 5, 24, 64
    q = np.stack([synth.integer_codes(rng, 2 * n, k) for _ in range(experts)])
    s = np.stack([synth.power_of_two_scales(rng, 2 * n, k // 32, lo=-6, hi=-3) for _ in range(experts)])
    packed = np.stack([oracle.pack(q[e]) for e in range(experts)])
    counts = [3, 0, 7, 1, 4]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    xs = synth.integer_activations(rng, int(sum(counts)), k)
    gate = oracle.grouped_linear(xs, packed[:, 0::2], s[:, 0::2], offsets, 32)
    up = oracle.grouped_linear(xs, packed[:, 1::2], s[:, 1::2], offsets, 32)
    got = oracle.grouped_swiglu_linear(xs, packed, s, offsets, 32)
    assert np.allclose(got, oracle.silu(gate) * up, rtol=1e-15, atol=0)


def test_moe_ffn_reduces_to_its_steps():
    """route -> grouped SwiGLU -> fp16 -> grouped down -> combine is the FFN."""
    rng = np.random.default_rng(9)
    experts, t_count, topk, hid, inter = 6, 11, 2, 64, 32
    gq = np.stack([synth.integer_codes(rng, 2 * inter, hid) for _ in range(experts)])
    gs = np.stack([synth.power_of_two_scales(rng, 2 * inter, hid // 32, lo=-8, hi=-5) for _ in range(experts)])
    dq = np.stack([synth.integer_codes(rng, hid, inter) for _ in range(experts)])
    ds = np.stack([synth.power_of_two_scales(rng, hid, inter // 32, lo=-6, hi=-3) for _ in range(experts)])
    gp = np.stack([oracle.pack(a) for a in gq])
    dp = np.stack([oracle.pack(a) for a in dq])
    x = synth.integer_activations(rng, t_count, hid)
    ids = np.stack([rng.choice(experts, topk, replace=False) for _ in range(t_count)])
    w = synth.router_weights(rng, t_count, topk)
    offsets, tok, slot, row = oracle.moe_route(ids, experts)
    h = oracle.grouped_swiglu_linear(x[tok], gp, gs, offsets, 32).astype(np.float16)
    yp = oracle.grouped_linear(h, dp, ds, offsets, 32)
    want = oracle.moe_combine(yp, row, w)
    assert np.allclose(oracle.moe_ffn(x, ids, w, gp, gs, dp, ds, 32), want, rtol=1e-13, atol=1e-13)

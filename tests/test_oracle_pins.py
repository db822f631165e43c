"""Pins for the fp64 oracle: facts fixed by the scheme and by mathematics.

The oracle is trusted only because these pass.  Each pin is written so that a
plausible mistake in the oracle (nibble order, offset, group index, transposed
operand, dropped group, wrong rounding of the scale) fails at least one of them;
``test_pins_catch_planted_mistakes`` plants such mistakes in copies of the
oracle's functions, on the CPU, and checks that the pins notice.

Scheme: int4 symmetric codes with one fp16 scale per group of 128 (32 for MoE)
along K and fp16 activations (LLM170, CUDA/W4A16 page, opening description);
kernel results must match a CPU reference of the quantised layer (same page,
Repository layout).
"""

import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Fixture readers.
# ---------------------------------------------------------------------------
def read_pack_words():
    rows = []
    for line in open(os.path.join(GOLDEN, "pack_words.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        rows.append(([int(v) for v in parts[:8]], int(parts[8], 16)))
    return rows


def read_quant_groups():
    groups = []
    cur = None
    for line in open(os.path.join(GOLDEN, "quantize_groups.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "group":
            cur = {"name": parts[1], "scale_bits": int(parts[3], 16), "w": [], "q": []}
            groups.append(cur)
        else:
            cur["w"].append(float(parts[0]))
            cur["q"].append(int(parts[1]))
    return groups


def real_impl():
    return types.SimpleNamespace(quantize=oracle.quantize, pack=oracle.pack, unpack=oracle.unpack,
                                 dequantize=oracle.dequantize, linear=oracle.linear)


# ---------------------------------------------------------------------------
# Pin checks, parameterised by implementation so planted mistakes can be run.
# Each returns None when the pin holds and raises AssertionError otherwise.
# ---------------------------------------------------------------------------
def pin_pack_golden(impl):
    for codes, word in read_pack_words():
        q = np.array([codes], dtype=np.int8)
        got = impl.pack(q)
        assert got.shape == (1, 1) and int(got[0, 0]) == word, (codes, hex(int(got[0, 0])), hex(word))
        back = impl.unpack(np.array([[word]], dtype=np.uint32))
        assert back.tolist() == [codes], (hex(word), back.tolist())


def pin_pack_roundtrip(impl):
    # every value at every position, others at 0
    for i in range(8):
        for v in range(-8, 8):
            q = np.zeros((1, 8), dtype=np.int8)
            q[0, i] = v
            assert impl.unpack(impl.pack(q)).tolist() == q.tolist()
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2 ** 32, size=(1000, 125), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(impl.pack(impl.unpack(words)), words)
    q = synth.integer_codes(rng, 37, 256)
    assert np.array_equal(impl.unpack(impl.pack(q)), q)


def pin_quantize_golden(impl):
    for g in read_quant_groups():
        w = np.zeros((1, 32), dtype=np.float32)
        want = np.zeros((1, 32), dtype=np.int8)
        w[0, : len(g["w"])] = g["w"]
        want[0, : len(g["q"])] = g["q"]
        q, s = impl.quantize(w, 32)
        assert int(np.asarray(s, dtype=np.float16).view(np.uint16)[0, 0]) == g["scale_bits"], g["name"]
        assert np.array_equal(q, want), (g["name"], q[0, : len(g["q"])].tolist(), g["q"])


def pin_quantize_invariants(impl):
    rng = np.random.default_rng(12)
    for group in (32, 128):
        w = synth.weights(rng, 64, 4 * group)
        w[3, :group] = 0.0                                       # an all-zero group
        w[5, group: 2 * group] *= 1e4                            # a large-scale group
        q, s = impl.quantize(w, group)
        assert q.dtype == np.int8 and s.dtype == np.float16
        assert q.min() >= -8 and q.max() <= 7
        assert q.min() >= -7, "s = fp16(max/7) keeps every code inside [-7, 7]"
        sf = np.repeat(s.astype(np.float64), group, axis=1)
        err = np.abs(w.astype(np.float64) - q.astype(np.float64) * sf)
        assert np.all(err <= sf / 2 * (1 + 1e-6) + 1e-30), float((err - sf / 2).max())
        assert s[3, 0] == 0 and np.all(q[3, :group] == 0)
        # the element of largest magnitude in every live group gets |q| = 7
        wg = np.abs(w.reshape(64, 4, group))
        amax = wg.argmax(axis=2)
        qg = np.abs(q.reshape(64, 4, group).astype(np.int64))
        live = s.astype(np.float64) > 0
        top = np.take_along_axis(qg, amax[..., None], axis=2)[..., 0]
        assert np.all(top[live] == 7)
        # the scale is the fp16 rounding of absmax / 7
        a = wg.max(axis=2).astype(np.float64) / 7.0
        rel = np.abs(s.astype(np.float64) - a) / np.where(a > 0, a, 1)
        assert np.all(rel[live] <= 2.0 ** -11 * 1.0001)


def pin_closed_forms(impl):
    # K = 128, one group.
    s = np.array([[2.0 ** -4]], dtype=np.float16)
    x1 = np.ones((1, 128), dtype=np.float16)
    q = np.full((1, 128), 7, dtype=np.int8)
    assert impl.linear(x1, impl.pack(q), s, 128).tolist() == [[56.0]]     # 128 * 7 / 16
    ramp = np.tile(np.arange(-8, 8, dtype=np.int8), 8)[None, :]
    s3 = np.array([[0.375]], dtype=np.float16)
    assert impl.linear(x1, impl.pack(ramp), s3, 128).tolist() == [[-64 * 0.375]]  # 8 * (-8) * s
    alt_q = np.tile(np.array([7, -7], dtype=np.int8), 64)[None, :]
    alt_x = np.tile(np.array([1, -1], dtype=np.float16), 64)[None, :]
    assert impl.linear(alt_x, impl.pack(alt_q), s3, 128).tolist() == [[896 * 0.375]]
    # one non-zero code at k0, two groups with different scales: checks nibble
    # position, group index and the sign/offset of the code.
    rng = np.random.default_rng(13)
    x = rng.integers(-3, 4, size=(2, 256)).astype(np.float16)
    x[x == 0] = 1
    s2 = np.array([[0.5, 0.125]], dtype=np.float16)
    for k0 in range(256):
        for v in (-8, -3, 5, 7):
            qq = np.zeros((1, 256), dtype=np.int8)
            qq[0, k0] = v
            y = impl.linear(x, impl.pack(qq), s2, 128)
            want = [[float(x[0, k0]) * v * float(s2[0, k0 // 128])],
                    [float(x[1, k0]) * v * float(s2[0, k0 // 128])]]
            assert y.tolist() == want, (k0, v, y.tolist(), want)
    # rows of W are outputs: row n carries one code at k = 5n (catches x . W vs x . W^T)
    n_out, k = 3, 128
    qq = np.zeros((n_out, k), dtype=np.int8)
    for n in range(n_out):
        qq[n, 5 * n] = n + 1
    x = np.arange(1, 4 * k + 1, dtype=np.float64).reshape(4, k).astype(np.float16) / np.float16(64)
    sone = np.ones((n_out, 1), dtype=np.float16)
    y = impl.linear(x, impl.pack(qq), sone, k)
    want = np.array([[float(x[m, 5 * n]) * (n + 1) for n in range(n_out)] for m in range(4)])
    assert y.shape == (4, n_out) and np.array_equal(y, want)


def pin_exact_integer_family(impl):
    """x integers, q integers, s = 2^e: y equals exact rational arithmetic."""
    rng = np.random.default_rng(14)
    for group in (32, 128):
        m, n, k = 3, 5, 512
        x = synth.integer_activations(rng, m, k)
        q = synth.integer_codes(rng, n, k)
        s = synth.power_of_two_scales(rng, n, k // group)
        y = impl.linear(x, impl.pack(q), s, group)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(int(x[i, kk])) * int(q[j, kk]) * Fraction(float(s[j, kk // group]))
                            for kk in range(k))
                assert Fraction(y[i, j]) == exact, (group, i, j)


def pin_scale_linearity(impl):
    rng = np.random.default_rng(15)
    group = 32
    w = synth.weights(rng, 6, 4 * group)
    x = synth.activations(rng, 2, 4 * group)
    q, s = impl.quantize(w, group)
    packed = impl.pack(q)
    y = impl.linear(x, packed, s, group)
    # scaling every scale by 2^j scales y by exactly 2^j
    for j in (-3, 1, 4):
        s2 = (s.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(impl.linear(x, packed, s2, group), y * 2.0 ** j)
    # doubling the scale of group g of row n adds exactly that group's share to y[:, n]
    for n, g in ((0, 0), (3, 2), (5, 3)):
        s_only = np.zeros_like(s)
        s_only[n, g] = s[n, g]
        share = impl.linear(x, packed, s_only, group)[:, n]
        s_dbl = s.copy()
        s_dbl[n, g] = np.float16(2 * float(s[n, g]))
        y2 = impl.linear(x, packed, s_dbl, group)
        np.testing.assert_allclose(y2[:, n], y[:, n] + share, rtol=1e-12, atol=1e-15)
        others = [c for c in range(6) if c != n]
        assert np.array_equal(y2[:, others], y[:, others])


PINS = [pin_pack_golden, pin_pack_roundtrip, pin_quantize_golden, pin_quantize_invariants,
        pin_closed_forms, pin_exact_integer_family, pin_scale_linearity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(real_impl())


# ---------------------------------------------------------------------------
# The library routine and the explicit loops agree.
# ---------------------------------------------------------------------------
def test_matmul_equals_explicit_loops():
    rng = np.random.default_rng(16)
    for group, (m, n, k) in ((32, (3, 4, 64)), (128, (2, 3, 256))):
        w = synth.weights(rng, n, k)
        x = synth.activations(rng, m, k)
        q, s = oracle.quantize(w, group)
        p = oracle.pack(q)
        np.testing.assert_allclose(oracle.linear(x, p, s, group), oracle.linear_loops(x, p, s, group),
                                   rtol=1e-12, atol=1e-14)


def test_rows_and_cols_are_slices_of_full():
    rng = np.random.default_rng(17)
    w = synth.weights(rng, 40, 256)
    x = synth.activations(rng, 6, 256)
    q, s = oracle.quantize(w, 128)
    p = oracle.pack(q)
    y = oracle.linear(x, p, s, 128)
    assert np.array_equal(oracle.linear_rows(x, p, s, 128, [5, 0, 3]), y[[5, 0, 3]])
    assert np.array_equal(oracle.linear_cols(x, p, s, 128, [39, 1, 7]), y[:, [39, 1, 7]])


def test_batched_rows_are_independent():
    """Row m of an M = 4 product equals the M = 1 product on x[m]."""
    rng = np.random.default_rng(18)
    w = synth.weights(rng, 33, 384)
    x = synth.activations(rng, 4, 384)
    q, s = oracle.quantize(w, 128)
    p = oracle.pack(q)
    y = oracle.linear(x, p, s, 128)
    for m in range(4):
        assert np.array_equal(oracle.linear(x[m: m + 1], p, s, 128), y[m: m + 1])


# ---------------------------------------------------------------------------
# Grouped (MoE) product.
# ---------------------------------------------------------------------------
def _small_moe(rng, experts=6, tokens=20, topk=3, n=16, k=64, group=32, skew=False):
    ws = [synth.weights(rng, n, k) for _ in range(experts)]
    x = synth.activations(rng, tokens, k)
    r = (synth.route_skewed if skew else synth.route_uniform)(rng, tokens, experts, topk)
    qs = [oracle.quantize(w, group) for w in ws]
    packed = np.stack([oracle.pack(q) for q, _ in qs])
    scales = np.stack([s for _, s in qs])
    return x, r, packed, scales


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(19)
    x, r, packed, scales = _small_moe(rng)
    xs = x[r.pair_token]
    y = oracle.grouped_linear(xs, packed, scales, r.offsets, 32)
    for i in range(len(r.pair_token)):
        e, t = r.pair_expert[i], r.pair_token[i]
        assert np.array_equal(y[i], oracle.linear(x[t: t + 1], packed[e], scales[e], 32)[0])


def test_grouped_expert_permutation_invariance():
    """Relabelling experts (and re-sorting rows) leaves each pair's output unchanged."""
    rng = np.random.default_rng(20)
    x, r, packed, scales = _small_moe(rng, skew=True)
    y = oracle.grouped_linear(x[r.pair_token], packed, scales, r.offsets, 32)
    perm = rng.permutation(packed.shape[0])            # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    new_e = perm[r.pair_expert]
    order = np.lexsort((r.pair_token, new_e))
    counts = np.bincount(new_e, minlength=packed.shape[0])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y2 = oracle.grouped_linear(x[r.pair_token[order]], packed[inv], scales[inv], offs, 32)
    assert np.array_equal(y2, y[order])


def test_grouped_empty_experts_and_validation():
    rng = np.random.default_rng(21)
    x, r, packed, scales = _small_moe(rng, experts=8, tokens=4, topk=2)
    assert (r.counts == 0).any()
    y = oracle.grouped_linear(x[r.pair_token], packed, scales, r.offsets, 32)
    assert y.shape == (8, 16)
    with pytest.raises(ValueError):
        oracle.grouped_linear(x[r.pair_token], packed, scales, r.offsets[::-1].copy(), 32)
    empty = oracle.grouped_linear(np.zeros((0, 64), np.float16), packed, scales, np.zeros(9, np.int32), 32)
    assert empty.shape == (0, 16)


# ---------------------------------------------------------------------------
# The tolerance check itself.
# ---------------------------------------------------------------------------
def test_compare_accepts_and_rejects():
    rng = np.random.default_rng(22)
    ref = rng.standard_normal((4, 300))
    assert oracle.compare(ref.astype(np.float16), ref)
    bad = ref.astype(np.float16).astype(np.float64)
    bad[2, 7] = np.nan
    assert not oracle.compare(bad, ref)
    bad = ref.copy()
    bad[1, 11] += 5e-3 * np.abs(ref).max()
    rep = oracle.compare(bad, ref)
    assert not rep and rep.first_bad == (1, 11)
    bad = ref.copy()
    bad[3] *= 1 + 3e-3                                   # row rel-L2 3e-3 > 1e-3
    rep = oracle.compare(bad, ref)
    assert not rep and rep.first_bad[0] == 3
    assert oracle.compare(np.zeros((0, 5)), np.zeros((0, 5)))


# ---------------------------------------------------------------------------
# Planted mistakes (CPU only): each mutant of the oracle must fail some pin.
# ---------------------------------------------------------------------------
def _mut_unpack_high_first(words):
    q = oracle.unpack(words)
    return q.reshape(*q.shape[:-1], -1, 8)[..., ::-1].reshape(q.shape)


def _mut_pack_high_first(q):
    q = np.asarray(q)
    return oracle.pack(q.reshape(*q.shape[:-1], -1, 8)[..., ::-1].reshape(q.shape))


def _mut_unpack_offset7(words):
    return (oracle.unpack(words).astype(np.int16) + 1).clip(-8, 7).astype(np.int8)


def _mut_dequant_group_mod(q, s, group):
    q = np.asarray(q)
    groups = s.shape[-1]
    idx = np.arange(q.shape[-1]) % groups                      # k % G instead of k // g
    return q.astype(np.float64) * s.astype(np.float64)[..., idx]


def _mut_dequant_drop_last_group(q, s, group):
    wd = oracle.dequantize(q, s, group)
    wd[..., -group:] = 0
    return wd


def _mut_quantize_exact_scale(w, group):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    q = np.zeros((n, k), np.int8)
    s = np.zeros((n, k // group), np.float16)
    for g in range(k // group):
        blk = w[:, g * group:(g + 1) * group]
        a = np.abs(blk).max(axis=1).astype(np.float64) / 7
        s[:, g] = a.astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(a[:, None] > 0, blk / np.where(a[:, None] > 0, a[:, None], 1), 0)
        q[:, g * group:(g + 1) * group] = np.clip(np.rint(r), -8, 7)
    return q, s


def _mut_quantize_round_half_away(w, group):
    q, s = oracle.quantize(w, group)
    w = np.asarray(w, np.float32)
    sf = np.repeat(s.astype(np.float32), group, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sf > 0, w / np.where(sf > 0, sf, 1), 0)
    return np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -8, 7).astype(np.int8), s


def _linear_with(dequant=None, unpack=None):
    dq = dequant or oracle.dequantize
    up = unpack or oracle.unpack

    def lin(x, packed, s, group):
        wd = dq(up(packed), s, group)
        return np.asarray(x, np.float16).astype(np.float64) @ wd.T
    return lin


def _mut_linear_transposed(x, packed, s, group):
    wd = oracle.dequantize(oracle.unpack(packed), s, group)
    x64 = np.asarray(x, np.float16).astype(np.float64)
    if wd.shape[0] == wd.shape[1]:
        return x64 @ wd
    return (x64 @ wd.T)[:, ::-1]                               # columns in the wrong order


def _mut_linear_fp32(x, packed, s, group):
    wd = oracle.dequantize(oracle.unpack(packed), s, group).astype(np.float32)
    return (np.asarray(x, np.float16).astype(np.float32) @ wd.T.astype(np.float32)).astype(np.float64)


MUTANTS = {
    "unpack_high_nibble_first": dict(unpack=_mut_unpack_high_first,
                                     linear=_linear_with(unpack=_mut_unpack_high_first)),
    "pack_high_nibble_first": dict(pack=_mut_pack_high_first),
    "unpack_offset_7": dict(unpack=_mut_unpack_offset7, linear=_linear_with(unpack=_mut_unpack_offset7)),
    "dequant_group_k_mod_G": dict(dequantize=_mut_dequant_group_mod,
                                  linear=_linear_with(dequant=_mut_dequant_group_mod)),
    "dequant_drops_last_group": dict(dequantize=_mut_dequant_drop_last_group,
                                     linear=_linear_with(dequant=_mut_dequant_drop_last_group)),
    "quantize_divides_by_exact_scale": dict(quantize=_mut_quantize_exact_scale),
    "quantize_rounds_half_away": dict(quantize=_mut_quantize_round_half_away),
    "linear_transposed_operand": dict(linear=_mut_linear_transposed),
    "linear_in_fp32": dict(linear=_mut_linear_fp32),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    impl = real_impl()
    for attr, fn in MUTANTS[name].items():
        setattr(impl, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_manifest_matches():
    """tests/manifest.json records the seeds, shapes and parity bars actually in use."""
    import importlib.util
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("write_manifest", os.path.join(here, "write_manifest.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(here, "manifest.json")) as f:
        assert json.load(f) == json.loads(json.dumps(mod.manifest()))

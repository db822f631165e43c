"""MoE grouped GEMM parity against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_bit_exact, assert_close, dev, host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    torch_mod()
    import w4a16_int4_weight_linear_amd as w4
    return w4


def run_grouped(w4, xs, packed, scales, offsets, group):
    y = w4.grouped_gemm(dev(xs), dev(packed), dev(scales), dev(np.asarray(offsets, np.int32)), group)
    torch_mod().cuda.synchronize()
    return host(y)


def exact_bank(rng, experts, n, k, group):
    q = np.stack([synth.integer_codes(rng, n, k) for _ in range(experts)])
    s = np.stack([synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3) for _ in range(experts)])
    return q, s


def offsets_from_counts(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# (experts, n, k, group, counts): empty experts, a single row, > 32 rows (several
# passes), ragged n, a K tail (k % 128 != 0), both group sizes.
EXACT_CASES = [
    (4, 256, 128, 32, [3, 0, 17, 1]),
    (3, 260, 384, 128, [33, 2, 65]),        # odd scales per row (3): per-chunk scale loads
    (3, 300, 256, 128, [40, 0, 5]),
    (5, 64, 2080, 32, [0, 0, 70, 2, 33]),
    (2, 512, 2048, 32, [1, 29]),
    (1, 100, 96, 32, [9]),
]


@pytest.mark.parametrize("experts,n,k,group,counts", EXACT_CASES)
def test_grouped_exact_integer_family(w4, experts, n, k, group, counts):
    rng = np.random.default_rng(7000 + experts + n + k)
    q, s = exact_bank(rng, experts, n, k, group)
    rows = int(sum(counts))
    xs = synth.integer_activations(rng, rows, k)
    offs = offsets_from_counts(counts)
    packed = np.stack([w4.pack(q[e]) for e in range(experts)])
    y = run_grouped(w4, xs, packed, s, offs, group)
    y_ref = oracle.grouped_linear(xs, np.stack([oracle.pack(q[e]) for e in range(experts)]), s, offs, group)
    assert_bit_exact(y, y_ref, f"E={experts} n={n} k={k} g={group} counts={counts}")


def test_grouped_all_rows_one_expert_and_skew(w4):
    rng = np.random.default_rng(7100)
    experts, n, k = 16, 512, 1024
    q, s = exact_bank(rng, experts, n, k, 32)
    packed = np.stack([w4.pack(q[e]) for e in range(experts)])
    p_ref = np.stack([oracle.pack(q[e]) for e in range(experts)])
    for counts in ([0] * 7 + [300] + [0] * 8, list(np.random.default_rng(1).zipf(1.5, experts).clip(0, 200))):
        offs = offsets_from_counts(counts)
        xs = synth.integer_activations(rng, int(offs[-1]), k)
        y = run_grouped(w4, xs, packed, s, offs, 32)
        assert_bit_exact(y, oracle.grouped_linear(xs, p_ref, s, offs, 32), f"counts={counts}")


def test_grouped_moe_workload_full_size(w4):
    """256 experts of [512 x 2048] g32, 512 tokens routed top-8: every output checked."""
    case = synth.MOE_CASES["moe_256e_512x2048_g32_top8"]
    ws, x, r = synth.moe_inputs(case)
    packed = np.empty((case.experts, case.n, case.k // 8), np.uint32)
    scales = np.empty((case.experts, case.n, case.k // case.group), np.float16)
    p_ref = np.empty_like(packed)
    s_ref = np.empty_like(scales)
    for e, w in enumerate(ws):
        packed[e], scales[e] = w4.quantize(w, case.group)
        q, s_ref[e] = oracle.quantize(w, case.group)
        p_ref[e] = oracle.pack(q)
    del ws
    assert np.array_equal(packed, p_ref) and np.array_equal(scales.view(np.uint16), s_ref.view(np.uint16))
    xs = x[r.pair_token]
    y = run_grouped(w4, xs, packed, scales, r.offsets, case.group)
    rep = assert_close(y, oracle.grouped_linear(xs, p_ref, s_ref, r.offsets, case.group), case.name)
    print(f"{case.name}: {rep.message}")


def test_grouped_equals_dense_per_expert_and_permutation(w4):
    rng = np.random.default_rng(7200)
    experts, n, k = 8, 384, 2048
    ws = [synth.weights(rng, n, k) for _ in range(experts)]
    pq = [w4.quantize(w, 32) for w in ws]
    packed = np.stack([p for p, _ in pq])
    scales = np.stack([s for _, s in pq])
    r = synth.route_skewed(rng, 100, experts, 3)
    x = synth.activations(rng, 100, k)
    xs = x[r.pair_token]
    y = run_grouped(w4, xs, packed, scales, r.offsets, 32)
    for e in range(experts):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            yd = host(w4.gemm(dev(xs[lo:hi]), dev(packed[e]), dev(scales[e]), 32))
            assert_close(y[lo:hi], yd.astype(np.float64), f"expert {e}")
    # relabel experts: each pair's output is bit-identical
    perm = rng.permutation(experts)
    inv = np.argsort(perm)
    new_e = perm[r.pair_expert]
    order = np.lexsort((r.pair_token, new_e))
    offs2 = offsets_from_counts(np.bincount(new_e, minlength=experts))
    y2 = run_grouped(w4, x[r.pair_token[order]], packed[inv], scales[inv], offs2, 32)
    assert np.array_equal(y2.view(np.uint16), y[order].view(np.uint16))
    y3 = run_grouped(w4, xs, packed, scales, r.offsets, 32)
    assert np.array_equal(y3.view(np.uint16), y.view(np.uint16))


def test_grouped_many_experts_work_item_scan(w4):
    """More than 256 experts (the device-side work-item scan takes several rounds of
    256), with empty experts, single rows, and experts of 32, 33 and 97 rows (one,
    two and four 32-row work items) spread over all rounds."""
    rng = np.random.default_rng(7300)
    experts, n, k = 700, 64, 256
    counts = np.zeros(experts, np.int64)
    picks = rng.choice(experts, 120, replace=False)
    counts[picks] = rng.integers(1, 6, size=120)
    counts[[0, 255, 256, 511, 512, 699]] = [32, 33, 97, 1, 64, 40]
    q, s = exact_bank(rng, experts, n, k, 32)
    offs = offsets_from_counts(counts)
    xs = synth.integer_activations(rng, int(offs[-1]), k)
    packed = np.stack([w4.pack(q[e]) for e in range(experts)])
    y = run_grouped(w4, xs, packed, s, offs, 32)
    y_ref = oracle.grouped_linear(xs, np.stack([oracle.pack(q[e]) for e in range(experts)]), s, offs, 32)
    assert_bit_exact(y, y_ref, f"E={experts} rows={int(offs[-1])}")


@pytest.mark.parametrize("group,k", [(32, 2048), (128, 2304)])
def test_grouped_scales_at_two_byte_offset(w4, group, k):
    """A scale bank 2 bytes past a 16-byte boundary takes the 2-byte scale loads, bit-exact."""
    torch = torch_mod()
    rng = np.random.default_rng(7400 + group)
    experts, n, counts = 3, 300, [5, 0, 40]
    q, s = exact_bank(rng, experts, n, k, group)
    xs = synth.integer_activations(rng, int(sum(counts)), k)
    offs = offsets_from_counts(counts)
    flat = torch.zeros(s.size + 8, dtype=torch.float16, device="cuda")
    sd = flat[1:1 + s.size].view(s.shape)
    sd.copy_(torch.from_numpy(s))
    assert sd.data_ptr() % 16 == 2
    packed = np.stack([w4.pack(q[e]) for e in range(experts)])
    y = host(w4.grouped_gemm(dev(xs), dev(packed), sd, dev(offs), group))
    y_ref = oracle.grouped_linear(xs, np.stack([oracle.pack(q[e]) for e in range(experts)]), s, offs, group)
    assert_bit_exact(y, y_ref, f"offset scales g={group}")

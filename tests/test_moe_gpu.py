"""The routed-expert steps on the GPU (routing permute, gathered grouped product,
router-weighted combine) against the fp64 oracle, through the C ABI."""

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


def route(w4, ids, experts):
    offs, tok, row = w4.moe_route(dev(np.ascontiguousarray(ids, dtype=np.int32)), experts)
    torch_mod().cuda.synchronize()
    return host(offs), host(tok), host(row)


def check_routing(ids, experts, offs, tok, row):
    """Offsets are unique and must equal the oracle's; the rows inside an expert may
    come in any order, so the rest is checked for validity."""
    ref_offs, _, _, _ = oracle.moe_route(ids, experts)
    assert np.array_equal(offs.astype(np.int64), ref_offs)
    p = ids.size
    assert sorted(row.ravel().tolist()) == list(range(p))
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            r, e = row[t, j], ids[t, j]
            assert tok[r] == t and offs[e] <= r < offs[e + 1]


@pytest.mark.parametrize("tokens,topk,experts", [(1, 1, 1), (37, 3, 300), (200, 6, 5000), (700, 2, 4)])
def test_route_matches_oracle(w4, tokens, topk, experts):
    rng = np.random.default_rng(9000 + tokens + experts)
    ids = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])
    check_routing(ids, experts, *route(w4, ids, experts))


def test_route_moe_workload_and_invalid_ids(w4):
    case = synth.MOE_CASES["moe_256e_512x2048_g32_top8"]
    rng = np.random.default_rng(case.seed)
    for _ in range(case.experts):           # the case's draw order: weights first, then x, then routing
        synth.weights(rng, 1, 1)
    r = synth.route_uniform(np.random.default_rng(9100), case.tokens, case.experts, case.topk)
    offs, tok, row = route(w4, r.choice, case.experts)
    check_routing(r.choice, case.experts, offs, tok, row)
    assert np.array_equal(offs, r.offsets)
    # ids outside [0, E) get no row and are not counted
    ids = np.array([[0, 5], [-1, 2], [7, 1]], np.int32)
    offs, tok, row = route(w4, ids, 6)
    assert row[1, 0] == -1 and row[2, 0] == -1 and offs[-1] == 4
    valid = ids[(ids >= 0) & (ids < 6)]
    assert np.array_equal(np.diff(offs), np.bincount(valid, minlength=6))


def test_gathered_grouped_product_bit_exact(w4):
    rng = np.random.default_rng(9200)
    experts, n, k, tokens, topk = 12, 300, 1024, 90, 3
    q = np.stack([synth.integer_codes(rng, n, k) for _ in range(experts)])
    s = np.stack([synth.power_of_two_scales(rng, n, k // 32, lo=-6, hi=-3) for _ in range(experts)])
    x = synth.integer_activations(rng, tokens, k)
    ids = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])
    offs, tok, row = route(w4, ids, experts)
    packed = np.stack([w4.pack(q[e]) for e in range(experts)])
    y = host(w4.grouped_gemm_gather(dev(x), dev(tok), dev(packed), dev(s), dev(offs), 32))
    y_ref = oracle.grouped_linear(x[tok], np.stack([oracle.pack(q[e]) for e in range(experts)]), s, offs, 32)
    assert_bit_exact(y, y_ref, "gathered grouped product")
    # the same bits as the grouped product on an explicitly sorted copy
    y2 = host(w4.grouped_gemm(dev(x[tok]), dev(packed), dev(s), dev(offs), 32))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("n", [512, 100])
def test_combine_bit_exact(w4, n):
    rng = np.random.default_rng(9300 + n)
    tokens, topk = 64, 4
    rows = tokens * topk
    y_pairs = rng.integers(-64, 65, size=(rows, n)).astype(np.float16)
    row = rng.permutation(rows).reshape(tokens, topk).astype(np.int32)
    w = np.ldexp(1.0, rng.integers(-3, 2, size=(tokens, topk))).astype(np.float32)
    w[::5] *= -1
    row[3, 1] = -1                          # a pair without a row contributes nothing
    out = host(w4.moe_combine(dev(y_pairs), dev(row), dev(w)))
    ref_row = row.astype(np.int64).copy()
    ref_w = w.copy()
    ref_w[3, 1] = 0.0
    ref_row[3, 1] = 0
    assert_bit_exact(out, oracle.moe_combine(y_pairs, ref_row, ref_w), f"combine n={n}")


def test_moe_layer_full_size(w4):
    """The 35B-A3B-like layer end to end on the GPU: route, gathered grouped product,
    router-weighted combine; every output checked against the layer's definition."""
    case = synth.MOE_CASES["moe_256e_512x2048_g32_top8"]
    ws, x, r = synth.moe_inputs(case)
    packed = np.empty((case.experts, case.n, case.k // 8), np.uint32)
    scales = np.empty((case.experts, case.n, case.k // case.group), np.float16)
    p_ref, s_ref = np.empty_like(packed), np.empty_like(scales)
    for e, w in enumerate(ws):
        packed[e], scales[e] = w4.quantize(w, case.group)
        qe, s_ref[e] = oracle.quantize(w, case.group)
        p_ref[e] = oracle.pack(qe)
    del ws
    wts = synth.router_weights(np.random.default_rng(case.seed + 500), case.tokens, case.topk)
    torch = torch_mod()
    ids_t = dev(r.choice)
    offs, tok, row = w4.moe_route(ids_t, case.experts)
    y_pairs = w4.grouped_gemm_gather(dev(x), tok, dev(packed), dev(scales), offs, case.group)
    out = host(w4.moe_combine(y_pairs, row, dev(wts)))
    torch.cuda.synchronize()
    rep = assert_close(out, oracle.moe_layer(x, r.choice, wts, p_ref, s_ref, case.group), "MoE layer")
    print(f"MoE layer: {rep.message}")

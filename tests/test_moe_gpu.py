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


# ---------------------------------------------------------------------------
# The experts' whole feed-forward: fused gate/up + SwiGLU, down projection, combine.
# ---------------------------------------------------------------------------
def _packed_banks(w4, q):
    """(library-packed, oracle-packed) words of an int8 code bank [E, n, k]."""
    lib = np.stack([w4.pack(q[e]) for e in range(q.shape[0])])
    ref = np.stack([oracle.pack(q[e]) for e in range(q.shape[0])])
    return lib, ref


@pytest.mark.parametrize("experts,n,k,group,counts", [
    (4, 96, 256, 32, [3, 0, 21, 40]),
    (3, 100, 384, 128, [1, 33, 7]),          # n even but not a multiple of 4: scalar stores
    (5, 512, 2048, 32, [16, 5, 0, 29, 64]),  # the expert gate/up shape (2 x 512 rows, K = 2048)
])
def test_grouped_swiglu_sorted_and_gathered(w4, experts, n, k, group, counts):
    rng = np.random.default_rng(7600 + n + k)
    q = synth.code_bank(rng, experts, 2 * n, k)
    s = synth.scale_bank(rng, experts, 2 * n, k // group)
    p, p_ref = _packed_banks(w4, q)
    rows = int(sum(counts))
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tokens = 50
    x = synth.activations(rng, tokens, k)
    tok = rng.integers(0, tokens, size=rows).astype(np.int32)
    y_ref = oracle.grouped_swiglu_linear(x[tok], p_ref, s, offs, group)
    y1 = host(w4.grouped_gemm_swiglu(dev(x[tok]), dev(p), dev(s), dev(offs), group))
    assert_close(y1, y_ref, f"sorted E={experts} n={n} k={k}")
    y2 = host(w4.grouped_gemm_swiglu(dev(x), dev(p), dev(s), dev(offs), group, pair_token=dev(tok)))
    assert_close(y2, y_ref, f"gathered E={experts} n={n} k={k}")
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_grouped_swiglu_gate_roles(w4):
    """Zero gate scales give exact zeros (SiLU(0) = 0) whatever the up rows hold; zero
    up scales likewise: the even rows are the gate, the odd rows the up projection."""
    rng = np.random.default_rng(7700)
    experts, n, k, counts = 3, 64, 256, [5, 17, 2]
    q = synth.code_bank(rng, experts, 2 * n, k)
    s = synth.scale_bank(rng, experts, 2 * n, k // 32)
    p, _ = _packed_banks(w4, q)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.activations(rng, int(sum(counts)), k)
    for zero_rows in (0, 1):
        s0 = s.copy()
        s0[:, zero_rows::2] = 0
        y = host(w4.grouped_gemm_swiglu(dev(x), dev(p), dev(s0), dev(offs), 32))
        assert not np.any(y.view(np.uint16) & 0x7FFF), f"rows {zero_rows}::2 zeroed"


def test_expert_down_projection_full_size(w4):
    """The experts' down projection (K = 512 -> N = 2048, g32) at the full 256-expert,
    4096-pair shape, bit-exact on the integer family."""
    rng = np.random.default_rng(7800)
    r = synth.route_uniform(rng, 512, 256, 8)
    q = rng.integers(-8, 8, size=(256, 2048, 512), dtype=np.int8)
    s = synth.power_of_two_scales(rng, 256 * 2048, 512 // 32, lo=-6, hi=-3).reshape(256, 2048, 16)
    p, p_ref = _packed_banks(w4, q)
    xs = synth.integer_activations(rng, len(r.pair_token), 512)
    y = host(w4.grouped_gemm(dev(xs), dev(p), dev(s), dev(r.offsets), 32))
    assert_bit_exact(y, oracle.grouped_linear(xs, p_ref, s, r.offsets, 32), "expert down 256 x [2048, 512]")


def run_moe_ffn(w4, x, ids, wts, gu, gus, dn, dns, experts, group, inter):
    """route -> gathered gate/up + SwiGLU -> down -> combine, all on the device."""
    offs, tok, row = w4.moe_route(ids, experts)
    h = w4.grouped_gemm_swiglu(x, gu, gus, offs, group, pair_token=tok)
    yp = w4.grouped_gemm(h, dn, dns, offs, group)
    return w4.moe_combine(yp, row, wts)


def test_moe_ffn_full_size(w4):
    """The routed experts' whole FFN at the 35B-A3B-like shape (256 experts, hidden 2048,
    intermediate 512, top-8 of 512 tokens, g32) against the oracle's moe_ffn, every output."""
    case = synth.FFN_CASES["moe_ffn_256e_h2048_i512_g32_top8"]
    gu_q, gu_s, dn_q, dn_s, x, r, wts = synth.moe_ffn_inputs(case)
    gu, gu_ref = _packed_banks(w4, gu_q)
    dn, dn_ref = _packed_banks(w4, dn_q)
    del gu_q, dn_q
    out = run_moe_ffn(w4, dev(x), dev(r.choice.astype(np.int32)), dev(wts), dev(gu), dev(gu_s), dev(dn), dev(dn_s),
                      case.experts, case.group, case.inter)
    y = host(out)
    ref = oracle.moe_ffn(x, r.choice, wts, gu_ref, gu_s, dn_ref, dn_s, case.group)
    rep = assert_close(y, ref, "moe ffn full size")
    print(f"moe ffn: {rep.message}")

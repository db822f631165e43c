"""Fused gate/up SwiGLU product parity against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, dev, host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    torch_mod()
    import w4a16_int4_weight_linear_amd as w4
    return w4


def gate_up_sides(w4, rng, n, k, group):
    """Gaussian gate and up weights quantised by each side, interleaved row by row."""
    wg, wu = synth.weights(rng, n, k), synth.weights(rng, n, k)
    (pg, sg), (pu, su) = w4.quantize(wg, group), w4.quantize(wu, group)
    qg, sgr = oracle.quantize(wg, group)
    qu, sur = oracle.quantize(wu, group)
    p = w4.interleave_rows(pg, pu)
    s = w4.interleave_rows(sg, su)
    p_ref = np.empty_like(p); p_ref[0::2], p_ref[1::2] = oracle.pack(qg), oracle.pack(qu)
    s_ref = np.empty_like(s); s_ref[0::2], s_ref[1::2] = sgr, sur
    return (p, s), (p_ref, s_ref)


def run(w4, x, p, s, group):
    y = w4.gemv_swiglu(dev(x), dev(p), dev(s), group)
    torch_mod().cuda.synchronize()
    return host(y)


# (m, n outputs, k, group): ragged n, a K tail inside a line, odd scale counts,
# partial activation chunks, both group sizes, 1 to 4 rows (the decode GEMV with
# the gate/up epilogue: odd pair counts, fewer pairs than CUs, a K long enough to
# need more workgroups than CUs, and one too long for their LDS staging, which
# falls back to the weight-streaming kernel) and 9 / 16 rows (that kernel).
CASES = [(1, 300, 2080, 32), (2, 777, 1536, 128), (3, 129, 640, 32), (4, 1000, 5120, 128), (1, 17, 384, 128),
         (4, 301, 16384, 128), (2, 5, 8192, 32), (1, 64, 65536, 128),
         (16, 17, 384, 128), (9, 2049, 6144, 32), (16, 512, 2048, 128)]


@pytest.mark.parametrize("m,n,k,group", CASES)
def test_swiglu_gaussian(w4, m, n, k, group):
    rng = np.random.default_rng(8000 + m + n + k)
    (p, s), (p_ref, s_ref) = gate_up_sides(w4, rng, n, k, group)
    x = synth.activations(rng, m, k)
    y = run(w4, x, p, s, group)
    assert_close(y, oracle.swiglu_linear(x, p_ref, s_ref, group), f"m={m} n={n} k={k} g={group}")


def test_swiglu_27b_gate_up_full_size(w4):
    """The 27B FFN's gate and up projections (2 x 17408 rows, K = 5120, g128) at M = 4, every output checked."""
    rng = np.random.default_rng(8100)
    (p, s), (p_ref, s_ref) = gate_up_sides(w4, rng, 17408, 5120, 128)
    x = synth.activations(rng, 4, 5120)
    y = run(w4, x, p, s, 128)
    rep = assert_close(y, oracle.swiglu_linear(x, p_ref, s_ref, 128), "27B gate/up")
    print(f"27B gate/up M=4: {rep.message}")


def test_swiglu_27b_gate_up_decode_full_size(w4):
    """The same gate/up pair at M = 1 (one decode token), every output checked."""
    rng = np.random.default_rng(8150)
    (p, s), (p_ref, s_ref) = gate_up_sides(w4, rng, 17408, 5120, 128)
    x = synth.activations(rng, 1, 5120)
    y = run(w4, x, p, s, 128)
    rep = assert_close(y, oracle.swiglu_linear(x, p_ref, s_ref, 128), "27B gate/up M=1")
    print(f"27B gate/up M=1: {rep.message}")


@pytest.mark.parametrize("m", [1, 3])
def test_swiglu_exact_zeros_decode(w4, m):
    """Integer codes and power-of-two scales on the decode path: zero ups give exact zeros, repeated calls agree bit for bit."""
    rng = np.random.default_rng(8250 + m)
    n, k = 333, 2048
    q = synth.integer_codes(rng, 2 * n, k)
    s = synth.power_of_two_scales(rng, 2 * n, k // 32, lo=-6, hi=-3)
    x = synth.activations(rng, m, k)
    p = w4.pack(q)
    s_up0 = s.copy(); s_up0[1::2] = 0
    assert np.all(run(w4, x, p, s_up0, 32).astype(np.float64) == 0)
    y1, y2 = run(w4, x, p, s, 32), run(w4, x, p, s, 32)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    assert_close(y1, oracle.swiglu_linear(x, oracle.pack(q), s, 32), f"integer family m={m}")


def test_swiglu_exact_zeros_and_determinism(w4):
    rng = np.random.default_rng(8200)
    n, k = 640, 1024
    q = synth.integer_codes(rng, 2 * n, k)
    s = synth.power_of_two_scales(rng, 2 * n, k // 128, lo=-6, hi=-3)
    x = synth.activations(rng, 5, k)
    p = w4.pack(q)
    s_up0 = s.copy(); s_up0[1::2] = 0        # up = 0 -> SiLU(g) * 0
    assert np.all(run(w4, x, p, s_up0, 128).astype(np.float64) == 0)
    s_g0 = s.copy(); s_g0[0::2] = 0          # gate = 0 -> SiLU(0) = 0
    assert np.all(run(w4, x, p, s_g0, 128).astype(np.float64) == 0)
    y1, y2 = run(w4, x, p, s, 128), run(w4, x, p, s, 128)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    assert_close(y1, oracle.swiglu_linear(x, oracle.pack(q), s, 128), "integer family")

"""Prefill GEMM parity against the fp64 oracle, through the C ABI.

Integer activations, codes and power-of-two scales make every MFMA product and
partial sum exact, so those outputs must equal the oracle's fp16 rounding bit
for bit; Gaussian inputs must meet the tolerances of oracle.check.  The
full-size prefill workloads run in the same launch configuration the
benchmark times and are checked on sampled full rows.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_bit_exact, assert_close, dev, gaussian_sides, host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    torch_mod()
    import w4a16_int4_weight_linear_amd as w4
    return w4


def run_gemm(w4, x, packed, scales, group):
    y = w4.gemm(dev(x), dev(packed), dev(scales), group)
    torch_mod().cuda.synchronize()
    return host(y)


# (m, n, k, group): one row, ragged M/N tiles, a K tail of 32 (K % 64 != 0),
# several K steps, both group sizes.
# The last two have more tiles than the 256 persistent workgroups: a full
# data-parallel round plus a stream-K remainder (264 and 260 tiles of 128 x 256).
EXACT_SHAPES = [(1, 64, 128, 128), (7, 300, 256, 32), (128, 256, 512, 128), (130, 260, 1024, 32),
                (257, 513, 5120, 128), (64, 100, 96, 32), (300, 1000, 2080, 32), (512, 17408 // 8, 640, 128),
                (1024, 8448, 256, 128), (640, 13312, 160, 32),
                # 256-row tiles (M >= 1024): ragged M and N, a K tail of 32 (g32), unaligned scale rows
                (1100, 700, 2080, 32), (2048, 513, 640, 128), (1030, 260, 384, 128)]


@pytest.mark.parametrize("m,n,k,group", EXACT_SHAPES)
def test_gemm_exact_integer_family(w4, m, n, k, group):
    rng = np.random.default_rng(5000 + m + n + k + group)
    x = synth.integer_activations(rng, m, k)
    q = synth.integer_codes(rng, n, k)
    s = synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3)
    y = run_gemm(w4, x, w4.pack(q), s, group)
    assert_bit_exact(y, oracle.linear(x, oracle.pack(q), s, group), f"m={m} n={n} k={k} g={group}")


@pytest.mark.parametrize("m,n,k,group", [(512, 1024, 2048, 128), (333, 777, 1280, 32), (4, 4096, 5120, 128)])
def test_gemm_gaussian(w4, m, n, k, group):
    rng = np.random.default_rng(6000 + m)
    w = synth.weights(rng, n, k)
    x = synth.activations(rng, m, k)
    (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, group)
    y = run_gemm(w4, x, p, s, group)
    assert_close(y, oracle.linear(x, p_ref, s_ref, group), f"m={m} n={n} k={k} g={group}")


@pytest.mark.parametrize("name", ["gemm_512x5120x17408_g128", "gemm_4096x5120x17408_g128"])
def test_gemm_workload_full_size(w4, name):
    """The prefill workloads at full size, in the launch the benchmark times,
    every output compared with the oracle (every tile, stream-K ones included)."""
    case = synth.DENSE_CASES[name]
    w, x = synth.dense_inputs(case)
    (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, case.group)
    del w
    y = run_gemm(w4, x, p, s, case.group)
    assert np.isfinite(y).all()
    rep = assert_close(y, oracle.linear(x, p_ref, s_ref, case.group), name)
    print(f"{name}: {rep.message}")


def test_gemm_matches_gemv_for_small_m(w4):
    """Two independent kernels on the same problem agree within the oracle's bars:
    six rows run on the GEMM kernel, rows 0-3 and 4-5 on the GEMV kernels."""
    rng = np.random.default_rng(6100)
    w = synth.weights(rng, 2000, 3072)
    x = synth.activations(rng, 6, 3072)
    p, s = w4.quantize(w, 128)
    yg = run_gemm(w4, x, p, s, 128)
    yv = np.concatenate([host(w4.gemv(dev(x[:4]), dev(p), dev(s), 128)),
                         host(w4.gemv(dev(x[4:]), dev(p), dev(s), 128))])
    assert_close(yg, yv.astype(np.float64), "gemm vs gemv")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemm_small_m_runs_gemv_kernels(w4, m):
    """w4a16_gemm with m <= 4 gives the GEMV kernels' bits (it dispatches to them)."""
    rng = np.random.default_rng(6150 + m)
    w = synth.weights(rng, 1000, 2048)
    x = synth.activations(rng, m, 2048)
    p, s = w4.quantize(w, 128)
    yg = run_gemm(w4, x, p, s, 128)
    yv = host(w4.gemv(dev(x), dev(p), dev(s), 128))
    assert np.array_equal(yg.view(np.uint16), yv.view(np.uint16))


def test_gemm_deterministic(w4):
    rng = np.random.default_rng(6200)
    w = synth.weights(rng, 1500, 2048)
    x = synth.activations(rng, 300, 2048)
    p, s = w4.quantize(w, 32)
    xd, pd, sd = dev(x), dev(p), dev(s)
    y1 = host(w4.gemm(xd, pd, sd, 32))
    y2 = host(w4.gemm(xd, pd, sd, 32))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


# (m, n, k, group) for 5 <= m <= 32, the weight-streaming kernel (16 rows per pass): a K tail inside
# a line (96, 2080), a partial last activation chunk (2080, 5120, 6144), odd scale
# counts per row (2080 g32, 384 g128), tiny N (17: two workgroups), six 16-row
# blocks per workgroup (23040 rows over 256 workgroups), both group sizes.
SKINNY_SHAPES = [(5, 100, 96, 32), (8, 300, 2080, 32), (13, 1000, 5120, 128), (16, 257, 384, 128),
                 (16, 2049, 4096, 32), (11, 17, 6144, 128), (6, 23040, 512, 128),
                 (18, 700, 1024, 32), (32, 513, 2304, 128)]   # two 16-row passes (16 + 2, 16 + 16)


@pytest.mark.parametrize("m,n,k,group", SKINNY_SHAPES)
def test_gemm_skinny_exact_integer_family(w4, m, n, k, group):
    rng = np.random.default_rng(5500 + m + n + k + group)
    x = synth.integer_activations(rng, m, k)
    q = synth.integer_codes(rng, n, k)
    s = synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3)
    y = run_gemm(w4, x, w4.pack(q), s, group)
    assert_bit_exact(y, oracle.linear(x, oracle.pack(q), s, group), f"m={m} n={n} k={k} g={group}")


@pytest.mark.parametrize("m,n,k", [(16, 17408, 5120), (8, 5120, 17408)])
def test_gemm_skinny_gaussian_27b_shapes(w4, m, n, k):
    """Batched decode of 8 / 16 sequences on the 27B FFN's up / down shapes, every output checked."""
    rng = np.random.default_rng(5600 + m)
    w = synth.weights(rng, n, k)
    x = synth.activations(rng, m, k)
    (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, 128)
    y = run_gemm(w4, x, p, s, 128)
    rep = assert_close(y, oracle.linear(x, p_ref, s_ref, 128), f"m={m} n={n} k={k}")
    print(f"m={m} n={n} k={k}: {rep.message}")

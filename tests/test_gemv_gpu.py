"""GEMV (decode, 1 <= M <= 4) parity against the fp64 oracle, through the C ABI.

Bars: integer activations, codes and power-of-two scales give exact sums in
any order, so those outputs must match the oracle bit for bit; Gaussian inputs
must meet the per-element and per-row tolerances of oracle.check.
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


def run_gemv(w4, x, packed, scales, group):
    y = w4.gemv(dev(x), dev(packed), dev(scales), group)
    torch_mod().cuda.synchronize()
    return host(y)


# (n, k, group): several row counts (1 row, fewer rows than waves, ragged),
# K giving whole and ragged lane coverage (k/16 = 8, 64, 130, 320, 1088 pieces).
# The last three cut rows between waves: one 512-chunk row per workgroup shared
# by 8 or 16 waves, 2-3 rows per workgroup, and 19-20 one-item rows.
EXACT_SHAPES = [(1, 128, 128), (37, 1024, 32), (300, 5120, 128), (65, 384, 128), (130, 2080, 32),
                (2049, 2048, 32), (20, 17408, 128), (256, 16384, 128), (600, 5120, 32), (5000, 1024, 32)]


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k,group", EXACT_SHAPES)
def test_gemv_exact_integer_family(w4, m, n, k, group):
    rng = np.random.default_rng(1000 + 7 * m + n + k + group)
    x = synth.integer_activations(rng, m, k)
    q = synth.integer_codes(rng, n, k)
    s = synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3)
    packed = w4.pack(q)
    y_ref = oracle.linear(x, oracle.pack(q), s, group)
    y = run_gemv(w4, x, packed, s, group)
    assert_bit_exact(y, y_ref, f"m={m} n={n} k={k} g={group}")


def test_gemv_extreme_codes(w4):
    """All codes -8 or all +7 with the largest |x| of the integer family."""
    for code in (-8, 7):
        q = np.full((96, 1024), code, np.int8)
        x = np.full((4, 1024), 2, np.float16)
        x[1] = -2
        s = np.full((96, 8), 2.0 ** -6, np.float16)
        y = run_gemv(w4, x, w4.pack(q), s, 128)
        assert_bit_exact(y, oracle.linear(x, oracle.pack(q), s, 128), f"code {code}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_gaussian_small(w4, m):
    rng = np.random.default_rng(2000 + m)
    for n, k, group in ((1000, 3072, 128), (333, 1024, 32), (64, 640, 32)):
        w = synth.weights(rng, n, k)
        x = synth.activations(rng, m, k)
        (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, group)
        y = run_gemv(w4, x, p, s, group)
        assert_close(y, oracle.linear(x, p_ref, s_ref, group), f"m={m} n={n} k={k}")


@pytest.mark.parametrize("name", ["gemv_1x1024x1024_g128", "gemv_up_1x5120x17408_g128",
                                  "gemv_down_1x17408x5120_g128", "gemv_np4_4x5120x5120_g128",
                                  "gemv_np4_4x5120x17408_g128"])
def test_gemv_workload_full_size(w4, name):
    """The decode workloads at their full sizes, every output checked."""
    case = synth.DENSE_CASES[name]
    w, x = synth.dense_inputs(case)
    (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, case.group)
    assert np.array_equal(p, p_ref) and np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    y = run_gemv(w4, x, p, s, case.group)
    rep = assert_close(y, oracle.linear(x, p_ref, s_ref, case.group), name)
    print(f"{name}: {rep.message}")


def test_gemv_deterministic_and_stream(w4):
    torch = torch_mod()
    rng = np.random.default_rng(3000)
    w = synth.weights(rng, 4097, 5120)
    x = synth.activations(rng, 4, 5120)
    p, s = w4.quantize(w, 128)
    xd, pd, sd = dev(x), dev(p), dev(s)
    y1 = host(w4.gemv(xd, pd, sd, 128))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        y2 = w4.gemv(xd, pd, sd, 128, stream=stream)
    stream.synchronize()
    assert np.array_equal(y1.view(np.uint16), host(y2).view(np.uint16))


def test_gemv_empty_k_gives_zero(w4):
    torch = torch_mod()
    y = torch.full((2, 33), 7.0, dtype=torch.float16, device="cuda")
    x = torch.empty((2, 0), dtype=torch.float16, device="cuda")
    p = torch.empty((33, 0), dtype=torch.int32, device="cuda")
    s = torch.empty((33, 0), dtype=torch.float16, device="cuda")
    w4.gemv(x, p, s, 128, out=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_gemv_max_k_is_usable(w4):
    for m in (1, 4):
        kmax = w4.lib.w4a16_gemv_max_k(m, 128)
        assert kmax >= 17408, (m, kmax)
        k = (kmax // 128) * 128
        rng = np.random.default_rng(4000 + m)
        x = synth.integer_activations(rng, m, k, -1, 1)
        q = synth.integer_codes(rng, 8, k)
        s = np.full((8, k // 128), 2.0 ** -8, np.float16)
        y = run_gemv(w4, x, w4.pack(q), s, 128)
        assert_bit_exact(y, oracle.linear(x, oracle.pack(q), s, 128), f"m={m} k={k}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_beyond_lds_cap(w4, m):
    """K longer than the LDS-staged decode kernels take: w4a16_gemv runs the
    chunk-staged weight-streaming kernel instead, still bit-exact."""
    kmax = w4.lib.w4a16_gemv_max_k(m, 128)
    for k, group in ((kmax + 4096, 128), (kmax + 1024 + 32, 32)):
        k = k // group * group
        rng = np.random.default_rng(4100 + m + k)
        x = synth.integer_activations(rng, m, k, -1, 1)
        q = synth.integer_codes(rng, 37, k)
        s = synth.power_of_two_scales(rng, 37, k // group, lo=-9, hi=-8)
        y = run_gemv(w4, x, w4.pack(q), s, group)
        assert_bit_exact(y, oracle.linear(x, oracle.pack(q), s, group), f"m={m} k={k} g={group}")


def _offset_scales(s: np.ndarray):
    """The scales on the device at an address 2 bytes past a 16-byte boundary."""
    torch = torch_mod()
    flat = torch.zeros(s.size + 8, dtype=torch.float16, device="cuda")
    view = flat[1:1 + s.size].view(s.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(s)))
    assert view.data_ptr() % 16 == 2 and view.is_contiguous()
    return view


@pytest.mark.parametrize("m", [1, 2, 3, 4, 9, 200])
@pytest.mark.parametrize("k,group", [(2048, 32), (2304, 128), (5120, 128)])
def test_scales_at_two_byte_offset(w4, m, k, group):
    """Scales need only 2-byte alignment: a scale pointer 2 bytes past a 16-byte
    boundary takes the kernels' 2-byte scale loads (or aligned staging), bit-exact."""
    rng = np.random.default_rng(4200 + m + k + group)
    n = 300
    x = synth.integer_activations(rng, m, k)
    q = synth.integer_codes(rng, n, k)
    s = synth.power_of_two_scales(rng, n, k // group, lo=-6, hi=-3)
    y_ref = oracle.linear(x, oracle.pack(q), s, group)
    sd = _offset_scales(s)
    fn = w4.gemv if m <= 4 else w4.gemm
    y = host(fn(dev(x), dev(w4.pack(q)), sd, group))
    assert_bit_exact(y, y_ref, f"m={m} k={k} g={group}")

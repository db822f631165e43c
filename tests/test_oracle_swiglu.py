"""Pins of the oracle's gated (SwiGLU) product, independent of its own code:
closed forms of SiLU, the library sigmoid, the roles of the interleaved rows,
and an explicit-loop brute force on a tiny case."""

import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


def test_silu_closed_forms():
    # SiLU(0) = 0; sigmoid(ln 3) = 3/4, so SiLU(ln 3) = (3/4) ln 3 and SiLU(-ln 3) = -(1/4) ln 3
    l3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, l3, -l3]))
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * l3) <= 1e-15 and abs(got[2] + 0.25 * l3) <= 1e-15
    # SiLU(x) - SiLU(-x) = x for every x; SiLU(x) -> x and -> 0 in the tails
    xs = np.linspace(-30, 30, 121)
    assert np.allclose(oracle.silu(xs) - oracle.silu(-xs), xs, rtol=0, atol=1e-12)
    assert abs(oracle.silu(np.array([60.0]))[0] - 60.0) < 1e-20 and abs(oracle.silu(np.array([-60.0]))[0]) < 1e-24
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0 and np.isfinite(oracle.silu(np.array([-1000.0]))[0])


def test_silu_equals_library_sigmoid():
    g = np.random.default_rng(0).standard_normal(10000) * 6
    assert np.allclose(oracle.silu(g), g * expit(g), rtol=1e-14, atol=0)


def _tiny(rng, m, n, k, group):
    x = synth.integer_activations(rng, m, k)
    q = synth.integer_codes(rng, 2 * n, k)
    s = synth.power_of_two_scales(rng, 2 * n, k // group, lo=-6, hi=-3)
    return x, q, s


def test_swiglu_roles_of_interleaved_rows():
    rng = np.random.default_rng(1)
    x, q, s = _tiny(rng, 3, 5, 256, 128)
    z = oracle.linear(x, oracle.pack(q), s, 128)
    y = oracle.swiglu_linear(x, oracle.pack(q), s, 128)
    # even rows are the gate (through SiLU), odd rows the up projection (linear)
    assert np.allclose(y, z[:, 0::2] * expit(z[:, 0::2]) * z[:, 1::2], rtol=1e-13, atol=1e-13)
    # zero up scales -> exact zeros; zero gate scales -> SiLU(0) = 0 -> exact zeros
    s_up0 = s.copy(); s_up0[1::2] = 0
    assert np.all(oracle.swiglu_linear(x, oracle.pack(q), s_up0, 128) == 0)
    s_g0 = s.copy(); s_g0[0::2] = 0
    assert np.all(oracle.swiglu_linear(x, oracle.pack(q), s_g0, 128) == 0)
    # swapping the roles changes the result (the pin above would catch a swap)
    swapped = np.empty_like(q); swapped[0::2], swapped[1::2] = q[1::2], q[0::2]
    s_sw = np.empty_like(s); s_sw[0::2], s_sw[1::2] = s[1::2], s[0::2]
    assert not np.allclose(oracle.swiglu_linear(x, oracle.pack(swapped), s_sw, 128), y)
    with pytest.raises(ValueError):
        oracle.swiglu_linear(x, oracle.pack(q[:-1]), s[:-1], 128)


def test_swiglu_brute_force_loops():
    rng = np.random.default_rng(2)
    x, q, s = _tiny(rng, 2, 3, 64, 32)
    words = oracle.pack(q)
    y = oracle.swiglu_linear(x, words, s, 32)
    for mi in range(2):
        for i in range(3):
            acc = [0.0, 0.0]
            for role in (0, 1):
                r = 2 * i + role
                for kk in range(64):
                    u = (int(words[r, kk // 8]) >> (4 * (kk % 8))) & 0xF
                    acc[role] += float(x[mi, kk]) * float(s[r, kk // 32]) * (u - 8)
            want = acc[0] / (1.0 + math.exp(-acc[0])) * acc[1]
            assert abs(y[mi, i] - want) <= 1e-12 * max(1.0, abs(want))

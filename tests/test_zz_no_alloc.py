"""The allocation-free product (w4a16_gemm_noalloc), called through the C ABI,
against w4a16_gemm with a caller workspace on the same inputs: two calls in a
row on the library's shared scratch, the second smaller, both bit-identical to
w4a16_gemm (same kernels and schedule) and within the oracle's bars."""

import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, dev, gaussian_sides, host, torch_mod

pytestmark = pytest.mark.gpu


def _noalloc(w4, x, p, s, group):
    torch = torch_mod()
    m, k = x.shape
    n = p.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = w4.lib.w4a16_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                                   ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(y.data_ptr()), m, n, k, group, st)
    assert rc == w4.OK, w4.lib.w4a16_status_str(rc)
    return y


# (m, n, k, group): a full data-parallel round plus a stream-K remainder (264
# tiles), then a smaller problem of stream-K tiles only (40 tiles, K tail).
CALLS = [(1024, 8448, 1024, 128), (300, 2000, 2080, 32)]


def test_noalloc_matches_gemm_two_calls():
    torch = torch_mod()
    import w4a16_int4_weight_linear_amd as w4
    for i, (m, n, k, group) in enumerate(CALLS):
        rng = np.random.default_rng(9900 + i)
        w = synth.weights(rng, n, k)
        x = synth.activations(rng, m, k)
        (p, s), (p_ref, s_ref) = gaussian_sides(w4, w, group)
        xd, pd, sd = dev(x), dev(p), dev(s)
        assert w4.lib.w4a16_gemm_workspace_bytes(m, n, k, group) > 0     # the split-K path runs
        y_na = _noalloc(w4, xd, pd, sd, group)
        ws = w4.gemm_workspace(m, n, k, group)
        y_ws = w4.gemm(xd, pd, sd, group, workspace=ws)
        torch.cuda.synchronize()
        a, b = host(y_na), host(y_ws)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"call {i}: differs from w4a16_gemm"
        assert_close(a, oracle.linear(x, p_ref, s_ref, group), f"call {i} m={m} n={n} k={k}")

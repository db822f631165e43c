"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, its host quantiser and packing match the oracle bit for bit, and every
validation error is reported before anything is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import w4a16_int4_weight_linear_amd as w4

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "w4a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(w4.lib, name), name           # dlsym succeeds
        assert name in w4.SIGNATURES, name           # the binding knows its signature
    assert set(w4.SIGNATURES) == set(names)


def test_version_and_status_strings():
    assert w4.lib.w4a16_abi_version() == 2
    for s in range(9):
        assert w4.lib.w4a16_status_str(s).decode().startswith("W4A16_")
    assert b"unknown" in w4.lib.w4a16_status_str(99)


# ---------------------------------------------------------------------------
# Host quantiser / packing: bit-exact against the oracle.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("group", [32, 128])
def test_quantize_matches_oracle_bit_exact(group):
    rng = np.random.default_rng(100 + group)
    w = synth.weights(rng, 96, 8 * group)
    w[0, :group] = 0                                    # zero group
    w[1, group:2 * group] *= 1e-7                       # tiny / subnormal scales
    w[2, :group] *= 3e3                                 # large scales
    w[3, :group] = np.float32(0.25)                     # constant group
    p, s = w4.quantize(w, group)
    q_ref, s_ref = oracle.quantize(w, group)
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(p, oracle.pack(q_ref))


def test_quantize_golden_groups():
    import test_oracle_pins as pins
    for g in pins.read_quant_groups():
        w = np.zeros((1, 32), np.float32)
        w[0, : len(g["w"])] = g["w"]
        p, s = w4.quantize(w, 32)
        assert int(s.view(np.uint16)[0, 0]) == g["scale_bits"], g["name"]
        want = np.zeros((1, 32), np.int8)
        want[0, : len(g["q"])] = g["q"]
        assert np.array_equal(w4.unpack(p, 32), want), g["name"]


def test_scale_rounding_over_many_magnitudes():
    """The C++ fp32->fp16 rounding of a/7 agrees with numpy across the fp16 range."""
    rng = np.random.default_rng(101)
    e = rng.uniform(-30, 18, size=4000)
    a = (np.exp2(e) * rng.uniform(1, 2, size=e.size)).astype(np.float32)
    w = np.zeros((a.size, 32), np.float32)
    w[:, 5] = a
    w[:, 9] = -a * np.float32(0.37)
    with np.errstate(over="ignore"):
        keep = (a / np.float32(7)).astype(np.float16) < np.float16(np.inf)
    w = w[keep]
    p, s = w4.quantize(w, 32)
    q_ref, s_ref = oracle.quantize(w, 32)
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(p, oracle.pack(q_ref))


def test_quantize_errors_write_nothing():
    w = np.ones((2, 32), np.float32)
    w[1, 3] = np.nan
    packed = np.full((2, 4), 0xDEADBEEF, np.uint32)
    scales = np.full((2, 1), 7, np.uint16)
    st = w4.lib.w4a16_quantize(w.ctypes.data, 2, 32, 32, packed.ctypes.data, scales.ctypes.data)
    assert st == w4.ERR_RANGE
    assert np.all(packed == 0xDEADBEEF) and np.all(scales == 7)
    w = np.full((1, 32), 1e6, np.float32)               # 1e6 / 7 overflows fp16
    assert w4.lib.w4a16_quantize(w.ctypes.data, 1, 32, 32, packed.ctypes.data, scales.ctypes.data) == w4.ERR_RANGE
    assert w4.lib.w4a16_quantize(w.ctypes.data, 1, 32, 64, packed.ctypes.data, scales.ctypes.data) == w4.ERR_GROUP
    assert w4.lib.w4a16_quantize(w.ctypes.data, 1, 48, 32, packed.ctypes.data, scales.ctypes.data) == w4.ERR_SHAPE
    assert w4.lib.w4a16_quantize(None, 1, 32, 32, packed.ctypes.data, scales.ctypes.data) == w4.ERR_NULL
    assert w4.lib.w4a16_quantize(None, 0, 32, 32, None, None) == w4.OK


def test_pack_unpack_match_oracle():
    rng = np.random.default_rng(102)
    q = synth.integer_codes(rng, 50, 256)
    p = w4.pack(q)
    assert np.array_equal(p, oracle.pack(q))
    assert np.array_equal(w4.unpack(p, 256), q)
    words = rng.integers(0, 2 ** 32, size=(64, 100), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(w4.unpack(words, 800), oracle.unpack(words))
    import test_oracle_pins as pins
    for codes, word in pins.read_pack_words():
        assert int(w4.pack(np.array([codes], np.int8))[0, 0]) == word


def test_pack_errors():
    q = np.zeros((1, 8), np.int8)
    q[0, 2] = 8
    out = np.zeros((1, 1), np.uint32)
    assert w4.lib.w4a16_pack(q.ctypes.data, 1, 8, out.ctypes.data) == w4.ERR_RANGE
    q[0, 2] = -9
    assert w4.lib.w4a16_pack(q.ctypes.data, 1, 8, out.ctypes.data) == w4.ERR_RANGE
    assert w4.lib.w4a16_pack(q.ctypes.data, 1, 12, out.ctypes.data) == w4.ERR_SHAPE
    assert w4.lib.w4a16_pack(None, 1, 8, out.ctypes.data) == w4.ERR_NULL
    assert w4.lib.w4a16_unpack(None, 1, 8, q.ctypes.data) == w4.ERR_NULL
    assert w4.lib.w4a16_unpack(out.ctypes.data, -1, 8, q.ctypes.data) == w4.ERR_SHAPE


# ---------------------------------------------------------------------------
# Device entry points: validation runs before any HIP call, so these need no GPU.
# ---------------------------------------------------------------------------
A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)


def test_gemv_validation():
    g = w4.lib.w4a16_gemv
    assert g(A, A, A, A, 1, 64, 128, 64, None) == w4.ERR_GROUP
    assert g(A, A, A, A, 1, 64, 100, 32, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, 5, 64, 128, 128, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, -1, 64, 128, 128, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, 1, -64, 128, 128, None) == w4.ERR_SHAPE
    assert g(A, A, A, None, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(None, A, A, A, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(A, None, A, A, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(A, A, None, A, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(A + 8, A, A, A, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A + 4, A, A, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A, A + 1, A, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A, A, A + 2, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A, A, A, 1, 1 << 22, 1 << 12, 128, None) == w4.ERR_SHAPE   # > 2 GiB of packed weights
    # empty problems succeed without touching anything
    assert g(None, None, None, None, 0, 64, 128, 128, None) == w4.OK
    assert g(None, None, None, None, 1, 0, 128, 128, None) == w4.OK
    assert w4.lib.w4a16_gemv_max_k(0, 128) == 0 and w4.lib.w4a16_gemv_max_k(5, 128) == 0
    assert w4.lib.w4a16_gemv_max_k(1, 64) == 0


def test_gemm_validation():
    g = w4.lib.w4a16_gemm
    assert g(A, A, A, A, 8, 64, 128, 16, A, 0, None) == w4.ERR_GROUP
    assert g(A, A, A, A, 8, 64, 96, 128, A, 0, None) == w4.ERR_SHAPE
    assert g(A, A, A, None, 8, 64, 128, 128, A, 0, None) == w4.ERR_NULL
    assert g(A, A, A, A + 8, 8, 64, 128, 128, A, 0, None) == w4.ERR_ALIGN
    assert g(A, A, A, A, 8, 64, 128, 128, A + 4, 0, None) == w4.ERR_ALIGN
    assert g(None, None, None, None, 0, 64, 128, 128, None, 0, None) == w4.OK
    assert w4.lib.w4a16_gemm_workspace_bytes(8, 64, 100, 32) == 0
    st = w4.lib.w4a16_gemm_workspace_status
    assert st(None, 4096, None) == w4.ERR_NULL
    assert st(A + 4, 4096, None) == w4.ERR_ALIGN
    assert st(A, 255, None) == w4.ERR_WORKSPACE     # smaller than the status header
    assert b"TIMEOUT" in w4.lib.w4a16_status_str(w4.ERR_TIMEOUT)


def test_gemv_swiglu_validation():
    g = w4.lib.w4a16_gemv_swiglu
    assert g(A, A, A, A, 1, 64, 128, 64, None) == w4.ERR_GROUP
    assert g(A, A, A, A, 1, 64, 100, 32, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, 17, 64, 128, 128, None) == w4.ERR_SHAPE    # at most 16 rows
    assert g(A, A, A, A, 1, -64, 128, 128, None) == w4.ERR_SHAPE
    assert g(A, A, A, None, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(A, None, A, A, 1, 64, 128, 128, None) == w4.ERR_NULL
    assert g(A + 8, A, A, A, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A, A, A + 2, 1, 64, 128, 128, None) == w4.ERR_ALIGN
    assert g(A, A, A, A, 1, 1 << 21, 1 << 12, 128, None) == w4.ERR_SHAPE   # 2n rows: > 2 GiB of weights
    assert g(None, None, None, None, 0, 64, 128, 128, None) == w4.OK
    assert g(None, None, None, None, 1, 0, 128, 128, None) == w4.OK


def test_moe_validation():
    r = w4.lib.w4a16_moe_route
    assert r(A, 4, 0, 8, A, A, A, None) == w4.ERR_SHAPE          # topk >= 1
    assert r(A, 4, 2, 0, A, A, A, None) == w4.ERR_SHAPE          # at least one expert
    assert r(A, 4, 2, 40000, A, A, A, None) == w4.ERR_SHAPE      # counted in LDS
    assert r(A, -1, 2, 8, A, A, A, None) == w4.ERR_SHAPE
    assert r(A, 4, 2, 8, None, A, A, None) == w4.ERR_NULL
    assert r(None, 4, 2, 8, A, A, A, None) == w4.ERR_NULL
    assert r(A + 2, 4, 2, 8, A, A, A, None) == w4.ERR_ALIGN
    gg = w4.lib.w4a16_grouped_gemm_gather
    assert gg(A, A, A, A, A, A, 4, 16, 8, 64, 128, 48, None) == w4.ERR_GROUP
    assert gg(A, None, A, A, A, A, 4, 16, 8, 64, 128, 32, None) == w4.ERR_NULL
    assert gg(A, A + 2, A, A, A, A, 4, 16, 8, 64, 128, 32, None) == w4.ERR_ALIGN
    assert gg(A, A, A, A, A, A, 4, 16, -8, 64, 128, 32, None) == w4.ERR_SHAPE
    assert gg(None, None, None, None, None, None, 4, 0, 8, 64, 128, 32, None) == w4.OK
    c = w4.lib.w4a16_moe_combine
    assert c(A, A, A, A, 4, 0, 32, 64, None) == w4.ERR_SHAPE
    assert c(A, A, A, None, 4, 2, 32, 64, None) == w4.ERR_NULL
    assert c(A, A, A, A + 8, 4, 2, 32, 64, None) == w4.ERR_ALIGN
    assert c(None, None, None, None, 0, 2, 0, 64, None) == w4.OK


def test_interleave_rows():
    a = np.arange(12, dtype=np.uint32).reshape(3, 4)
    b = a + 100
    r = w4.interleave_rows(a, b)
    assert r.shape == (6, 4) and np.array_equal(r[0::2], a) and np.array_equal(r[1::2], b)
    with pytest.raises(ValueError):
        w4.interleave_rows(a, b[:2])


def test_grouped_validation():
    g = w4.lib.w4a16_grouped_gemm
    assert g(A, A, A, A, A, 4, 16, 64, 128, 48, None) == w4.ERR_GROUP
    assert g(A, A, A, A, A, 4, 16, 64, 100, 32, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, A, -1, 16, 64, 128, 32, None) == w4.ERR_SHAPE
    assert g(A, A, A, A, A, 0, 16, 64, 128, 32, None) == w4.ERR_SHAPE
    assert g(A, A, A, None, A, 4, 16, 64, 128, 32, None) == w4.ERR_NULL
    assert g(A, A, A, A, None, 4, 16, 64, 128, 32, None) == w4.ERR_NULL
    assert g(A, A, A, A + 2, A, 4, 16, 64, 128, 32, None) == w4.ERR_ALIGN
    assert g(A, A, A, A, A + 2, 4, 16, 64, 128, 32, None) == w4.ERR_ALIGN
    assert g(None, None, None, None, None, 4, 0, 64, 128, 32, None) == w4.OK


def test_binding_raises_on_error():
    with pytest.raises(w4.W4A16Error) as e:
        w4.quantize(np.ones((1, 48), np.float32), 32)
    assert e.value.status == w4.ERR_SHAPE


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The package has no fallback: without libw4a16.so the import itself fails."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "w4a16_int4_weight_linear_amd")
    pkg = tmp_path / "w4a16_int4_weight_linear_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(src, "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import w4a16_int4_weight_linear_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is missing" in r.stderr

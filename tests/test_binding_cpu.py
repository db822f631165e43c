"""The Python binding checks every tensor argument before it calls the library:
dtype, contiguity and shape, then that all tensors are on one HIP device.  A
mismatch raises ValueError (TypeError for a non-tensor) and nothing reaches the
C ABI, which only sees pointers.  CPU tensors are used here: every check below
fires before any device call, and a CPU tensor itself is refused by the last one.
"""

import pytest
import torch

import w4a16_int4_weight_linear_amd as w4


def dense(m=2, n=64, k=256, group=128):
    x = torch.zeros((m, k), dtype=torch.float16)
    p = torch.zeros((n, k // 8), dtype=torch.int32)
    s = torch.zeros((n, k // group), dtype=torch.float16)
    return x, p, s


@pytest.mark.parametrize("fn", [w4.gemv, w4.gemm])
def test_dense_checks(fn):
    x, p, s = dense()
    with pytest.raises(ValueError, match="dtype"):
        fn(x.float(), p, s, 128)
    with pytest.raises(ValueError, match="dtype"):
        fn(x, p.long(), s, 128)                       # int64 words
    with pytest.raises(ValueError, match="dtype"):
        fn(x, p, s.float(), 128)                      # fp32 scales
    with pytest.raises(ValueError, match="contiguous"):
        fn(torch.zeros((256, 2), dtype=torch.float16).t(), p, s, 128)
    with pytest.raises(ValueError, match="shape"):
        fn(x, p[:, :16].contiguous(), s, 128)         # packed words of a shorter k
    with pytest.raises(ValueError, match="shape"):
        fn(x, p, s[:32], 128)                         # scales of fewer rows
    with pytest.raises(ValueError, match="shape"):
        fn(x, p, s, 32)                               # scales of group 128, call says 32
    with pytest.raises(ValueError, match="multiple"):
        fn(x, p, s, 64)
    with pytest.raises(ValueError, match="2-D"):
        fn(x[0], p, s, 128)
    with pytest.raises(ValueError, match="shape"):
        fn(x, p, s, 128, out=torch.zeros((2, 63), dtype=torch.float16))
    with pytest.raises(ValueError, match="dtype"):
        fn(x, p, s, 128, out=torch.zeros((2, 64), dtype=torch.float32))
    with pytest.raises(TypeError):
        fn(x, p.numpy(), s, 128)
    with pytest.raises(ValueError, match="HIP device"):
        fn(x, p, s, 128)                              # everything right, but host memory


def test_gemm_workspace_checked():
    x, p, s = dense(m=64)
    with pytest.raises(ValueError, match="dtype"):
        w4.gemm(x, p, s, 128, workspace=torch.zeros(16, dtype=torch.float32))


def test_swiglu_checks():
    x, p, s = dense(n=64)
    with pytest.raises(ValueError, match="multiple of 2 rows"):
        w4.gemv_swiglu(x, p[:63], s[:63], 128)
    with pytest.raises(ValueError, match="shape"):
        w4.gemv_swiglu(x, p, s, 128, out=torch.zeros((2, 64), dtype=torch.float16))   # n = 32 outputs
    with pytest.raises(ValueError, match="HIP device"):
        w4.gemv_swiglu(x, p, s, 128)


def bank(e=4, n=64, k=256, group=32):
    return (torch.zeros((e, n, k // 8), dtype=torch.int32), torch.zeros((e, n, k // group), dtype=torch.float16),
            torch.zeros(e + 1, dtype=torch.int32))


def test_grouped_checks():
    p, s, off = bank()
    x = torch.zeros((10, 256), dtype=torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        w4.grouped_gemm(x, p, s, off.long(), 32)      # int64 offsets
    with pytest.raises(ValueError, match="shape"):
        w4.grouped_gemm(x, p, s, off[:4], 32)         # one offset short
    with pytest.raises(ValueError, match="shape"):
        w4.grouped_gemm(x, p, s[:, :, :4].contiguous(), off, 32)   # scales of another group size
    with pytest.raises(ValueError, match=r"\[experts"):
        w4.grouped_gemm(x, p[0], s, off, 32)
    with pytest.raises(ValueError, match="HIP device"):
        w4.grouped_gemm(x, p, s, off, 32)
    tok = torch.zeros(10, dtype=torch.int64)
    with pytest.raises(ValueError, match="dtype"):
        w4.grouped_gemm_gather(x, tok, p, s, off, 32)  # int64 token index (torch.topk's dtype)
    with pytest.raises(ValueError, match="HIP device"):
        w4.grouped_gemm_gather(x, tok.int(), p, s, off, 32)


def test_moe_route_and_combine_checks():
    with pytest.raises(ValueError, match="dtype"):
        w4.moe_route(torch.zeros((4, 2), dtype=torch.int64), 8)   # torch.topk returns int64
    with pytest.raises(ValueError, match="tokens, topk"):
        w4.moe_route(torch.zeros(8, dtype=torch.int32), 8)
    y = torch.zeros((8, 64), dtype=torch.float16)
    row = torch.zeros((4, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="dtype"):
        w4.moe_combine(y, row, torch.zeros((4, 2), dtype=torch.float16))   # fp16 router weights
    with pytest.raises(ValueError, match="shape"):
        w4.moe_combine(y, row, torch.zeros((4, 3), dtype=torch.float32))
    with pytest.raises(ValueError, match="HIP device"):
        w4.moe_combine(y, row, torch.zeros((4, 2), dtype=torch.float32))

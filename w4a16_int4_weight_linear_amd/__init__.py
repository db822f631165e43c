"""Python binding of the gfx950 W4A16 int4 weight-only linear layer (libw4a16.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels (device entry points) or its C++ host routines (quantise / pack).
PyTorch supplies device memory and the current HIP stream.  The C entry points
are exposed under their own names (``w4a16_gemv`` ...) on ``lib``; the
functions below wrap them for torch tensors.

The library must have been built (``python -m w4a16_int4_weight_linear_amd.build``
or ``__graft_entry__.build()``); importing without it raises ImportError, and
there is no fallback path of any kind.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -m w4a16_int4_weight_linear_amd.build)")

# PyTorch ships its own HIP runtime under the same soname as the system one.
# Whichever is loaded first serves the whole process, and torch's streams and
# allocations must come from the runtime the library uses, so torch (when it
# is installed) is imported before the library is loaded.
try:
    import torch as _torch_preload  # noqa: F401
except ImportError:  # no torch: the host routines (quantise / pack) still work
    _torch_preload = None

lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

# The entry points of include/w4a16.h with their C signatures.
SIGNATURES = {
    "w4a16_abi_version": (ctypes.c_int, []),
    "w4a16_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a16_quantize": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "w4a16_pack": (ctypes.c_int, [_vp, _i64, _i64, _vp]),
    "w4a16_unpack": (ctypes.c_int, [_vp, _i64, _i64, _vp]),
    "w4a16_gemv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "w4a16_gemv_max_k": (_i64, [_i64, _i32]),
    "w4a16_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "w4a16_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "w4a16_gemm_workspace_status": (ctypes.c_int, [_vp, _sz, _vp]),
    "w4a16_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "w4a16_hbm_read_probe": (ctypes.c_int, [_vp, _sz, _vp, _sz, _vp]),
    "w4a16_hbm_read_probe_sink_words": (_i64, []),
    "w4a16_grouped_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp]),
    "w4a16_gemv_swiglu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "w4a16_moe_route": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_grouped_gemm_gather": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i32,
                                                 _vp]),
    "w4a16_moe_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i64, _vp]),
    "w4a16_grouped_gemm_swiglu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i32,
                                                 _vp]),
}

for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args
    globals()[_name] = _fn

OK, ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_RANGE, ERR_TIMEOUT = range(9)


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.w4a16_status_str(status).decode()}")


def _check(status: int, what: str):
    if status != OK:
        raise W4A16Error(status, what)


# ---------------------------------------------------------------------------
# Host routines (numpy in, numpy out).
# ---------------------------------------------------------------------------
def quantize(w: np.ndarray, group: int):
    """fp32 w [n, k] -> (packed uint32 [n, k/8], scales fp16 [n, k/group])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    packed = np.empty((n, k // 8), dtype=np.uint32)
    scales = np.empty((n, k // group if group else 0), dtype=np.float16)
    _check(lib.w4a16_quantize(w.ctypes.data, n, k, group, packed.ctypes.data, scales.ctypes.data), "quantize")
    return packed, scales


def pack(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    out = np.empty((n, k // 8), dtype=np.uint32)
    _check(lib.w4a16_pack(q.ctypes.data, n, k, out.ctypes.data), "pack")
    return out


def unpack(packed: np.ndarray, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    n = packed.shape[0]
    out = np.empty((n, k), dtype=np.int8)
    _check(lib.w4a16_unpack(packed.ctypes.data, n, k, out.ctypes.data), "unpack")
    return out


# ---------------------------------------------------------------------------
# Device routines (torch tensors on the current HIP device).
#
# Every argument is checked before the C call: dtype, contiguity and shape
# first, then that every tensor lives on the same HIP device.  A mismatch
# raises ValueError (TypeError for a non-tensor) and nothing is launched, since
# the library itself can only check pointers, not what they point to.
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _dev_packed(packed):
    """uint32 words travel as torch.int32 (same bits)."""
    torch = _torch()
    if isinstance(packed, np.ndarray):
        packed = torch.from_numpy(np.ascontiguousarray(packed).view(np.int32))
    return packed


def _dtypes(kind):
    torch = _torch()
    return {
        "f16": (torch.float16,),
        "f32": (torch.float32,),
        "i32": (torch.int32,),
        # packed words: int32 or uint32 tensors (the same 32 bits)
        "u32": tuple(d for d in (torch.int32, getattr(torch, "uint32", None)) if d is not None),
    }[kind]


def _check_tensors(what, specs):
    """specs: (name, tensor, dtype kind, expected shape or None).  Raises before any launch."""
    torch = _torch()
    for name, t, kind, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}: {name} must be a torch.Tensor, not {type(t).__name__}")
        if t.dtype not in _dtypes(kind):
            raise ValueError(f"{what}: {name} has dtype {t.dtype}, expected {_dtypes(kind)[0]}")
        if not t.is_contiguous():
            raise ValueError(f"{what}: {name} must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    devs = {t.device for _, t, _, _ in specs}
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{what}: {name} is on {t.device}; every tensor must be on the HIP device")
    if len(devs) > 1:
        raise ValueError(f"{what}: tensors are on different devices {sorted(map(str, devs))}")


def _require_tensors(what, **tensors):
    torch = _torch()
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}: {name} must be a torch.Tensor, not {type(t).__name__}")


def _dense_shapes(what, x, packed, scales, group, rows_per_out=1):
    """(m, n, k, specs) of a dense product: the 2-D layouts checked, the tensor specs
    returned for _check_tensors; n counts output columns."""
    _require_tensors(what, x=x, packed=packed, scales=scales)
    if x.dim() != 2 or packed.dim() != 2 or scales.dim() != 2:
        raise ValueError(f"{what}: x, packed and scales must be 2-D")
    m, k = x.shape
    if group not in (32, 128) or k % group:
        raise ValueError(f"{what}: k = {k} must be a multiple of the group size 32 or 128 (got {group})")
    nw = packed.shape[0]
    if nw % rows_per_out:
        raise ValueError(f"{what}: packed must have a multiple of {rows_per_out} rows")
    specs = [("x", x, "f16", None), ("packed", packed, "u32", (nw, k // 8)),
             ("scales", scales, "f16", (nw, k // group))]
    return m, nw // rows_per_out, k, specs


def _checked_out(what, specs, out, shape, like):
    """Check specs plus the output (if given); returns the output, allocated if None."""
    torch = _torch()
    _check_tensors(what, specs + ([("out", out, "f16", shape)] if out is not None else []))
    if out is None:
        out = torch.empty(shape, dtype=torch.float16, device=like.device)
    return out


def gemv(x, packed, scales, group: int, out=None, stream=None):
    """y [m, n] fp16 = x [m, k] . deq(packed, scales)^T, 1 <= m <= 4."""
    m, n, k, specs = _dense_shapes("gemv", x, packed, scales, group)
    out = _checked_out("gemv", specs, out, (m, n), x)
    _check(lib.w4a16_gemv(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k, group, _stream(stream)),
           "w4a16_gemv")
    return out


def gemm_workspace(m: int, n: int, k: int, group: int, device=None):
    """A zero-filled workspace tensor of the size w4a16_gemm needs (None if none)."""
    torch = _torch()
    nbytes = lib.w4a16_gemm_workspace_bytes(m, n, k, group)
    if nbytes == 0:
        return None
    return torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device=device or "cuda")


# Workspaces gemm() keeps when the caller passes none: one per (device, stream),
# grown to the largest size asked for.  Calls on one stream run one after
# another, which is all a workspace needs; the library leaves it ready for reuse.
_WORKSPACES = {}


def _cached_workspace(m, n, k, group, device, stream_handle):
    torch = _torch()
    nbytes = lib.w4a16_gemm_workspace_bytes(m, n, k, group)
    if nbytes == 0:
        return None
    key = (str(device), stream_handle)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() * 4 < nbytes:
        ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device=device)
        _WORKSPACES[key] = ws
    return ws


def gemm(x, packed, scales, group: int, out=None, workspace=None, stream=None):
    """y [m, n] fp16 = x [m, k] . deq(packed, scales)^T for any m (fp16 MFMA, fp32 accumulate)."""
    m, n, k, specs = _dense_shapes("gemm", x, packed, scales, group)
    if workspace is not None:
        specs = specs + [("workspace", workspace, "i32", None)]
    out = _checked_out("gemm", specs, out, (m, n), x)
    st = _stream(stream)
    if workspace is None:
        workspace = _cached_workspace(m, n, k, group, x.device, st.value)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.w4a16_gemm(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k, group, _ptr(workspace),
                          ws_bytes, st), "w4a16_gemm")
    return out


def gemm_noalloc(x, packed, scales, group: int, out=None, stream=None):
    """gemm without a workspace: the library's own scratch holds the split-K partials
    (calls that overlap on one GPU race; allocates nothing when `out` is given)."""
    m, n, k, specs = _dense_shapes("gemm_noalloc", x, packed, scales, group)
    out = _checked_out("gemm_noalloc", specs, out, (m, n), x)
    _check(lib.w4a16_gemm_noalloc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k, group, _stream(stream)),
           "w4a16_gemm_noalloc")
    return out


def hbm_read_probe(buf, sink, stream=None):
    """Read all of `buf` (a device tensor, 1 KiB multiple) once; one XOR per wave goes to
    `sink` (int32, at least lib.w4a16_hbm_read_probe_sink_words() elements)."""
    _check_tensors("hbm_read_probe", [("sink", sink, "i32", None)])
    _check(lib.w4a16_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                    _stream(stream)), "w4a16_hbm_read_probe")


def gemm_workspace_status(workspace, stream=None) -> int:
    """Status word of a gemm workspace (host-synchronous diagnostic): OK, or ERR_TIMEOUT if a
    split-K fix-up of an earlier call gave up waiting (its tiles were written as NaN)."""
    _check_tensors("gemm_workspace_status", [("workspace", workspace, "i32", None)])
    return lib.w4a16_gemm_workspace_status(_ptr(workspace), workspace.numel() * 4, _stream(stream))


def interleave_rows(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """Rows of gate and up interleaved (gate row i -> 2i, up row i -> 2i + 1): the
    weight layout of gemv_swiglu, for packed words and scales alike."""
    gate, up = np.asarray(gate), np.asarray(up)
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    out = np.empty((2 * gate.shape[0],) + gate.shape[1:], dtype=gate.dtype)
    out[0::2], out[1::2] = gate, up
    return out


def gemv_swiglu(x, packed, scales, group: int, out=None, stream=None):
    """y [m, n] = SiLU(x . Wg^T) * (x . Wu^T), 1 <= m <= 16; packed [2n, k/8] interleaves gate/up rows."""
    m, n, k, specs = _dense_shapes("gemv_swiglu", x, packed, scales, group, rows_per_out=2)
    out = _checked_out("gemv_swiglu", specs, out, (m, n), x)
    _check(lib.w4a16_gemv_swiglu(_ptr(x), _ptr(packed), _ptr(scales), _ptr(out), m, n, k, group, _stream(stream)),
           "w4a16_gemv_swiglu")
    return out


def _bank_shapes(what, packed, scales, k, group):
    _require_tensors(what, packed=packed, scales=scales)
    if packed.dim() != 3 or scales.dim() != 3:
        raise ValueError(f"{what}: packed and scales must be [experts, n, ...]")
    if group not in (32, 128) or k % group:
        raise ValueError(f"{what}: k = {k} must be a multiple of the group size 32 or 128 (got {group})")
    experts, n = packed.shape[0], packed.shape[1]
    return experts, n, [("packed", packed, "u32", (experts, n, k // 8)),
                        ("scales", scales, "f16", (experts, n, k // group))]


def grouped_gemm(x, packed, scales, offsets, group: int, out=None, stream=None):
    """MoE grouped product: rows offsets[e]..offsets[e+1] of x use expert e's weights."""
    _require_tensors("grouped_gemm", x=x)
    if x.dim() != 2:
        raise ValueError("grouped_gemm: x must be [rows, k]")
    rows, k = x.shape
    experts, n, bank = _bank_shapes("grouped_gemm", packed, scales, k, group)
    out = _checked_out("grouped_gemm", [("x", x, "f16", None)] + bank + [("offsets", offsets, "i32", (experts + 1,))],
                       out, (rows, n), x)
    _check(lib.w4a16_grouped_gemm(_ptr(x), _ptr(packed), _ptr(scales), _ptr(offsets), _ptr(out), experts, rows,
                                  n, k, group, _stream(stream)), "w4a16_grouped_gemm")
    return out


def moe_route(topk_ids, experts: int, stream=None):
    """Device routing of int32 topk_ids [tokens, topk] -> (offsets [E+1], pair_token [P], pair_row [tokens, topk])."""
    _require_tensors("moe_route", topk_ids=topk_ids)
    torch = _torch()
    if topk_ids.dim() != 2:
        raise ValueError("moe_route: topk_ids must be [tokens, topk]")
    _check_tensors("moe_route", [("topk_ids", topk_ids, "i32", None)])
    t, topk = topk_ids.shape
    dev_ = topk_ids.device
    offsets = torch.empty(experts + 1, dtype=torch.int32, device=dev_)
    pair_token = torch.empty(t * topk, dtype=torch.int32, device=dev_)
    pair_row = torch.empty((t, topk), dtype=torch.int32, device=dev_)
    _check(lib.w4a16_moe_route(_ptr(topk_ids), t, topk, experts, _ptr(offsets), _ptr(pair_token), _ptr(pair_row),
                               _stream(stream)), "w4a16_moe_route")
    return offsets, pair_token, pair_row


def grouped_gemm_gather(x, pair_token, packed, scales, offsets, group: int, out=None, stream=None):
    """Grouped product whose row r reads token pair_token[r] of x [tokens, k]."""
    _require_tensors("grouped_gemm_gather", x=x, pair_token=pair_token)
    if x.dim() != 2 or pair_token.dim() != 1:
        raise ValueError("grouped_gemm_gather: x must be [tokens, k] and pair_token [rows]")
    tokens, k = x.shape
    rows = pair_token.shape[0]
    experts, n, bank = _bank_shapes("grouped_gemm_gather", packed, scales, k, group)
    out = _checked_out("grouped_gemm_gather", [("x", x, "f16", None), ("pair_token", pair_token, "i32", None)] +
                       bank + [("offsets", offsets, "i32", (experts + 1,))], out, (rows, n), x)
    _check(lib.w4a16_grouped_gemm_gather(_ptr(x), _ptr(pair_token), _ptr(packed), _ptr(scales), _ptr(offsets),
                                         _ptr(out), experts, rows, tokens, n, k, group, _stream(stream)),
           "w4a16_grouped_gemm_gather")
    return out


def grouped_gemm_swiglu(x, packed, scales, offsets, group: int, pair_token=None, out=None, stream=None):
    """Experts' fused gate/up + SwiGLU: packed [E, 2n, k/8] interleaves gate/up rows; y [rows, n].
    pair_token None: x [rows, k] is sorted by expert; else grouped row r reads x[pair_token[r]]."""
    _require_tensors("grouped_gemm_swiglu", x=x)
    if x.dim() != 2:
        raise ValueError("grouped_gemm_swiglu: x must be 2-D")
    x_rows, k = x.shape
    experts, n2, bank = _bank_shapes("grouped_gemm_swiglu", packed, scales, k, group)
    if n2 % 2:
        raise ValueError("grouped_gemm_swiglu: packed must have a multiple of 2 rows per expert")
    specs = [("x", x, "f16", None)] + bank + [("offsets", offsets, "i32", (experts + 1,))]
    if pair_token is not None:
        _require_tensors("grouped_gemm_swiglu", pair_token=pair_token)
        if pair_token.dim() != 1:
            raise ValueError("grouped_gemm_swiglu: pair_token must be [rows]")
        specs.append(("pair_token", pair_token, "i32", None))
        rows = pair_token.shape[0]
    else:
        rows = x_rows
    out = _checked_out("grouped_gemm_swiglu", specs, out, (rows, n2 // 2), x)
    _check(lib.w4a16_grouped_gemm_swiglu(_ptr(x), _ptr(pair_token), _ptr(packed), _ptr(scales), _ptr(offsets),
                                         _ptr(out), experts, rows, x_rows, n2 // 2, k, group, _stream(stream)),
           "w4a16_grouped_gemm_swiglu")
    return out


def moe_combine(y_pairs, pair_row, weights, out=None, stream=None):
    """out [tokens, n] = sum_j weights[t, j] * y_pairs[pair_row[t, j]] (weights fp32 [tokens, topk])."""
    _require_tensors("moe_combine", y_pairs=y_pairs, pair_row=pair_row, weights=weights)
    if y_pairs.dim() != 2 or pair_row.dim() != 2:
        raise ValueError("moe_combine: y_pairs must be [rows, n] and pair_row [tokens, topk]")
    tokens, topk = pair_row.shape
    rows, n = y_pairs.shape
    out = _checked_out("moe_combine", [("y_pairs", y_pairs, "f16", None), ("pair_row", pair_row, "i32", None),
                                       ("weights", weights, "f32", (tokens, topk))], out, (tokens, n), y_pairs)
    _check(lib.w4a16_moe_combine(_ptr(y_pairs), _ptr(pair_row), _ptr(weights), _ptr(out), tokens, topk, rows, n,
                                 _stream(stream)), "w4a16_moe_combine")
    return out


__all__ = ["lib", "LIB_PATH", "SIGNATURES", "W4A16Error", "quantize", "pack", "unpack", "gemv", "gemm",
           "gemm_workspace", "gemm_workspace_status", "gemm_noalloc",
           "hbm_read_probe", "grouped_gemm_swiglu", "grouped_gemm", "interleave_rows", "gemv_swiglu", "moe_route",
           "grouped_gemm_gather", "moe_combine"] + list(SIGNATURES)

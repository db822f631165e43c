"""Plain, slow, fp64 CPU reference for the W4A16 int4 weight-only linear layer.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

What is computed (LLM170, CUDA/W4A16 page, opening description): weights are
int4 and symmetric (no zero point) with one scale per group of ``g`` input
features along K (g = 128 for the dense model, 32 for the MoE models), and the
activations are IEEE binary16.  The same page (Repository layout) requires the
GPU kernels' outputs to match a CPU reference of the quantised layer; this is
that reference, written from the definition

    y[m, n] = sum_k x[m, k] * s[n, k // g] * q[n, k]

with x and s the exact fp16 values, q in [-8, 7] the stored code, everything
carried in fp64.  The pages fix nothing finer, so these readings are used
(each is listed in the design notes):

* quantiser: a = max |w| over the group (fp32), s = fp16(a / 7) with the
  division in fp32 and round-to-nearest-even to fp16; q = clamp(rint(w / s),
  -8, 7) with the division in fp32 and ties to even; s == 0 gives q = 0;
* storage: offset-binary nibble u = q + 8; eight nibbles per uint32 along K,
  element k = 8 j + i of a row in bits [4 i, 4 i + 4) of word j (low nibble
  first); packed weights are [N, K/8] uint32 row-major, scales [N, K/g] fp16;
* weight orientation: W is [N, K] (output x input), y = x . W^T;
* MoE: rows sorted by expert, rows of expert e are offsets[e]..offsets[e+1],
  one output row per (token, expert) pair, no combine.
"""

from __future__ import annotations

import numpy as np

GROUPS = (32, 128)


# ---------------------------------------------------------------------------
# Quantiser (scheme from the LLM170 CUDA/W4A16 page, opening description).
# ---------------------------------------------------------------------------
def quantize(w: np.ndarray, group: int):
    """Symmetric int4 quantisation of fp32 weights w [N, K] with one scale per group.

    Returns (q int8 [N, K] in [-8, 7], s float16 [N, K // group]).
    Raises ValueError for non-finite weights or scales that overflow fp16.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if group <= 0 or k % group:
        raise ValueError("K must be a multiple of the group size")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    q = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, k // group), dtype=np.float16)
    for gi in range(k // group):
        cols = slice(gi * group, (gi + 1) * group)
        block = w[:, cols]                                   # fp32 [N, g]
        a = np.max(np.abs(block), axis=1)                    # group absmax, fp32
        scale = (a / np.float32(7.0)).astype(np.float16)     # fp32 divide, RNE to fp16
        if not np.all(np.isfinite(scale)):
            raise ValueError("group scale overflows fp16")
        s[:, gi] = scale
        sf = scale.astype(np.float32)[:, None]
        live = sf[:, 0] != 0                                 # s == 0 (all-zero group or underflow): q = 0
        r = block[live] / sf[live]                           # fp32 divide
        q[live, cols] = np.clip(np.rint(r), -8, 7).astype(np.int8)
    return q, s


# ---------------------------------------------------------------------------
# Storage: eight offset-binary nibbles per uint32 along K, low nibble first.
# ---------------------------------------------------------------------------
def pack(q: np.ndarray) -> np.ndarray:
    """int8 codes [..., K] in [-8, 7] -> uint32 words [..., K/8]."""
    q = np.asarray(q)
    if q.shape[-1] % 8:
        raise ValueError("K must be a multiple of 8")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("code outside [-8, 7]")
    u = (q.astype(np.int64) + 8).astype(np.uint64)
    u = u.reshape(*q.shape[:-1], q.shape[-1] // 8, 8)
    words = np.zeros(u.shape[:-1], dtype=np.uint64)
    for i in range(8):
        words |= u[..., i] << np.uint64(4 * i)
    return words.astype(np.uint32)


def unpack(words: np.ndarray) -> np.ndarray:
    """uint32 words [..., K/8] -> int8 codes [..., K]."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    out = np.empty((*words.shape, 8), dtype=np.int8)
    for i in range(8):
        out[..., i] = ((words >> np.uint64(4 * i)) & np.uint64(0xF)).astype(np.int64) - 8
    return out.reshape(*words.shape[:-1], words.shape[-1] * 8)


def dequantize(q: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """W[n, k] = q[n, k] * s[n, k // group], exactly, in fp64."""
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float16)
    if q.shape[-1] != s.shape[-1] * group:
        raise ValueError("scale shape does not match K / group")
    return q.astype(np.float64) * np.repeat(s.astype(np.float64), group, axis=-1)


# ---------------------------------------------------------------------------
# The layer.
# ---------------------------------------------------------------------------
def linear(x: np.ndarray, packed: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """y [M, N] = x [M, K] . dequant(packed, s)^T, in fp64 (x is fp16)."""
    x = np.asarray(x, dtype=np.float16)
    wd = dequantize(unpack(packed), s, group)               # [N, K] fp64
    if x.shape[1] != wd.shape[1]:
        raise ValueError("x and W disagree on K")
    return x.astype(np.float64) @ wd.T


def linear_rows(x: np.ndarray, packed: np.ndarray, s: np.ndarray, group: int, rows) -> np.ndarray:
    """Only the listed rows of y, each full width: y[rows, :] (fp64)."""
    rows = np.asarray(rows, dtype=np.int64)
    return linear(np.asarray(x)[rows], packed, s, group)


def linear_cols(x: np.ndarray, packed: np.ndarray, s: np.ndarray, group: int, cols) -> np.ndarray:
    """Only the listed output columns of y, all rows: y[:, cols] (fp64)."""
    cols = np.asarray(cols, dtype=np.int64)
    return linear(x, np.asarray(packed)[cols], np.asarray(s)[cols], group)


def linear_loops(x: np.ndarray, packed: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """The definition as explicit Python loops over m, n, k (tiny shapes only)."""
    x = np.asarray(x, dtype=np.float16)
    words = np.asarray(packed, dtype=np.uint32)
    s = np.asarray(s, dtype=np.float16)
    m_dim, k_dim = x.shape
    n_dim = words.shape[0]
    y = np.zeros((m_dim, n_dim), dtype=np.float64)
    for m in range(m_dim):
        for n in range(n_dim):
            acc = 0.0
            for k in range(k_dim):
                u = (int(words[n, k // 8]) >> (4 * (k % 8))) & 0xF
                acc += float(x[m, k]) * float(s[n, k // group]) * (u - 8)
            y[m, n] = acc
    return y


def grouped_linear(x_sorted: np.ndarray, packed: np.ndarray, s: np.ndarray,
                   offsets: np.ndarray, group: int) -> np.ndarray:
    """MoE grouped product: for each expert e, y[r] = x_sorted[r] . W_e^T for r in its rows.

    packed [E, N, K/8], s [E, N, K/g], offsets int [E+1] (non-decreasing, 0..rows).
    """
    x_sorted = np.asarray(x_sorted, dtype=np.float16)
    offsets = np.asarray(offsets, dtype=np.int64)
    e_count = packed.shape[0]
    if offsets.shape != (e_count + 1,):
        raise ValueError("offsets must have E+1 entries")
    if offsets[0] != 0 or offsets[-1] != x_sorted.shape[0] or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must run non-decreasing from 0 to rows")
    y = np.zeros((x_sorted.shape[0], packed.shape[1]), dtype=np.float64)
    for e in range(e_count):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            y[lo:hi] = linear(x_sorted[lo:hi], packed[e], s[e], group)
    return y


# ---------------------------------------------------------------------------
# Gated feed-forward input (SwiGLU): the SiLU-activated gate projection times
# the up projection (rust-inference page, the "SwiGLU missing gate" item of
# its bug list), with the gate and up projections fused into one pass (infr
# page, Validated models & performance, footnote on Linear + GatedAct fusion).
# Reading: one weight tensor of 2N interleaved rows, row 2i the gate row of
# output i and row 2i + 1 its up row; SiLU(g) = g / (1 + e^-g).
# ---------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), in fp64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_linear(x: np.ndarray, packed: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """y [M, N] = SiLU(x . Wg^T) * (x . Wu^T), Wg / Wu the even / odd rows of the [2N, K] weights."""
    z = linear(x, packed, s, group)                          # [M, 2N] fp64
    if z.shape[1] % 2:
        raise ValueError("gate/up weights need an even number of rows")
    return silu(z[:, 0::2]) * z[:, 1::2]


# ---------------------------------------------------------------------------
# The routed-expert (MoE) layer around the grouped product: routing each token
# to its top-k experts, the experts' products, and the router-weighted combine
# back into one output row per token (the MoE tiles and the batched MoE path of
# the LLM170 / infr pages; the step either side of expert_gateup/expert_down).
# Readings: expert ids arrive as an int [T, topk] array; the grouped rows are
# ordered by (expert, token, slot); the combine is sum_j w[t, j] * y_pair(t, j)
# with the router weights w given (fp32), accumulated in fp64 here.
# ---------------------------------------------------------------------------
def moe_route(topk_ids: np.ndarray, experts: int):
    """(offsets int64 [E+1], pair_token int64 [P], pair_slot int64 [P], pair_row int64 [T, topk]).

    Sorted rows r = 0 .. P-1 list the (token, slot) pairs by (expert, token, slot);
    rows offsets[e] .. offsets[e+1]-1 belong to expert e; pair_row[t, j] is the row of (t, j).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    if ids.ndim != 2 or np.any(ids < 0) or np.any(ids >= experts):
        raise ValueError("expert ids must be an int [T, topk] array in [0, experts)")
    t_count, topk = ids.shape
    pairs = [(int(ids[t, j]), t, j) for t in range(t_count) for j in range(topk)]
    pairs.sort()
    offsets = np.zeros(experts + 1, dtype=np.int64)
    for e, _, _ in pairs:
        offsets[e + 1] += 1
    offsets = np.cumsum(offsets)
    pair_token = np.array([t for _, t, _ in pairs], dtype=np.int64)
    pair_slot = np.array([j for _, _, j in pairs], dtype=np.int64)
    pair_row = np.zeros((t_count, topk), dtype=np.int64)
    for r, (_, t, j) in enumerate(pairs):
        pair_row[t, j] = r
    return offsets, pair_token, pair_slot, pair_row


def moe_combine(y_pairs: np.ndarray, pair_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """out [T, N] = sum_j weights[t, j] * y_pairs[pair_row[t, j]], in fp64."""
    y_pairs = np.asarray(y_pairs, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    t_count, topk = w.shape
    out = np.zeros((t_count, y_pairs.shape[1]), dtype=np.float64)
    for t in range(t_count):
        for j in range(topk):
            out[t] += w[t, j] * y_pairs[pair_row[t, j]]
    return out


def moe_layer(x: np.ndarray, topk_ids: np.ndarray, weights: np.ndarray, packed: np.ndarray, s: np.ndarray,
              group: int) -> np.ndarray:
    """The routed-expert layer by its definition: out[t] = sum_j w[t, j] * (x[t] . W_{e(t, j)}^T), fp64."""
    x = np.asarray(x, dtype=np.float16)
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((x.shape[0], packed.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        ts, js = np.nonzero(ids == e)
        ye = linear(x[ts], packed[e], s[e], group)          # [pairs of e, N]
        for r in range(len(ts)):
            out[ts[r]] += w[ts[r], js[r]] * ye[r]
    return out


# ---------------------------------------------------------------------------
# The routed experts' feed-forward: each expert's fused gate/up projection with
# its SwiGLU activation, then its down projection, combined with the router
# weights (the expert_gateup / expert_down roles of the infr page's
# benchmarking section; SwiGLU as on the rust-inference page).  Reading: the
# SwiGLU output is the down projection's input activation, and activations are
# fp16 in the W4A16 scheme, so it is rounded to fp16 (nearest even) in between;
# everything else is fp64.
# ---------------------------------------------------------------------------
def grouped_swiglu_linear(x_sorted: np.ndarray, packed: np.ndarray, s: np.ndarray,
                          offsets: np.ndarray, group: int) -> np.ndarray:
    """Rows offsets[e]..offsets[e+1]-1 of x_sorted through expert e's interleaved gate/up
    rows: y[r] = SiLU(x[r] . Wg_e^T) * (x[r] . Wu_e^T), fp64 (packed [E, 2N, K/8])."""
    x_sorted = np.asarray(x_sorted, dtype=np.float16)
    offsets = np.asarray(offsets, dtype=np.int64)
    out = np.zeros((x_sorted.shape[0], packed.shape[1] // 2), dtype=np.float64)
    for e in range(packed.shape[0]):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = swiglu_linear(x_sorted[r0:r1], packed[e], s[e], group)
    return out


def moe_ffn(x: np.ndarray, topk_ids: np.ndarray, weights: np.ndarray, gu_packed: np.ndarray, gu_s: np.ndarray,
            dn_packed: np.ndarray, dn_s: np.ndarray, group: int) -> np.ndarray:
    """out[t] = sum_j w[t, j] * (h[t, j] . Wd_e^T), e = topk_ids[t, j], with
    h[t, j] = fp16(SiLU(x[t] . Wg_e^T) * (x[t] . Wu_e^T)); fp64 otherwise."""
    x = np.asarray(x, dtype=np.float16)
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((x.shape[0], dn_packed.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        ts, js = np.nonzero(ids == e)
        h = swiglu_linear(x[ts], gu_packed[e], gu_s[e], group).astype(np.float16)
        yd = linear(h, dn_packed[e], dn_s[e], group)
        for r in range(len(ts)):
            out[ts[r]] += w[ts[r], js[r]] * yd[r]
    return out

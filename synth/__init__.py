"""Seeded synthetic inputs for the W4A16 linear layer.

This module draws raw inputs only: fp32 Gaussian weights, fp16 Gaussian
activations, and the MoE routing of tokens to experts.  It holds none of the
layer's arithmetic (no quantisation, packing, scaling or products), so the
oracle and the GPU path can both start from exactly the same draws.

The workloads stand in for the layers of the models named on the LLM170 page
(CUDA/W4A16 era, opening description and benchmark tables): a 27B dense model
quantised with groups of 128 and a 35B-A3B mixture-of-experts model quantised
with groups of 32.  The pages print no layer dimensions, so the shapes below are
the stand-ins used throughout this repository:

* dense FFN: hidden 5120, intermediate 17408 (up projection K=5120, N=17408;
  down projection K=17408, N=5120), group 128;
* MoE: 256 experts of [512 x 2048] (N=512 outputs, K=2048 hidden), group 32,
  512 tokens each routed to 8 distinct experts drawn uniformly.

Every generator takes a seed and uses numpy's PCG64 (``default_rng``).  Within
one case the weights are drawn first, then the activations, then the routing.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02


def weights(rng: np.random.Generator, n: int, k: int, std: float = WEIGHT_STD) -> np.ndarray:
    """fp32 weights [n, k] ~ N(0, std^2) (row n = output feature n)."""
    return rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)


def activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """fp16 activations [m, k]: N(0, 1) drawn in fp32, cast to fp16 (round to nearest even)."""
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


@dataclass
class DenseCase:
    name: str
    seed: int
    m: int
    n: int
    k: int
    group: int


@dataclass
class MoECase:
    name: str
    seed: int
    tokens: int
    experts: int
    topk: int
    n: int
    k: int
    group: int


# Dense workloads.  Names say what each one is; the seed recipe is stated in
# the design notes and is the only thing that makes two runs draw the same data.
DENSE_CASES = {
    "gemv_1x1024x1024_g128": DenseCase("gemv_1x1024x1024_g128", 1, 1, 1024, 1024, 128),
    "gemv_up_1x5120x17408_g128": DenseCase("gemv_up_1x5120x17408_g128", 2, 1, 17408, 5120, 128),
    "gemv_down_1x17408x5120_g128": DenseCase("gemv_down_1x17408x5120_g128", 3, 1, 5120, 17408, 128),
    "gemv_np4_4x5120x5120_g128": DenseCase("gemv_np4_4x5120x5120_g128", 4, 4, 5120, 5120, 128),
    "gemv_np4_4x5120x17408_g128": DenseCase("gemv_np4_4x5120x17408_g128", 5, 4, 17408, 5120, 128),
    "gemm_512x5120x17408_g128": DenseCase("gemm_512x5120x17408_g128", 6, 512, 17408, 5120, 128),
    "gemm_4096x5120x17408_g128": DenseCase("gemm_4096x5120x17408_g128", 6, 4096, 17408, 5120, 128),
}

MOE_CASES = {
    "moe_256e_512x2048_g32_top8": MoECase("moe_256e_512x2048_g32_top8", 7, 512, 256, 8, 512, 2048, 32),
}


@dataclass
class MoEFFNCase:
    name: str
    seed: int
    tokens: int
    experts: int
    topk: int
    hidden: int        # the layer's input and output width (gate/up K, down N)
    inter: int         # the expert's intermediate width (gate/up outputs, down K)
    group: int


# The routed experts' whole feed-forward at the 35B-A3B-like shape: per expert a
# fused gate/up projection [2 x 512, 2048] and a down projection [2048, 512], g32.
FFN_CASES = {
    "moe_ffn_256e_h2048_i512_g32_top8": MoEFFNCase("moe_ffn_256e_h2048_i512_g32_top8", 8, 512, 256, 8, 2048, 512, 32),
}


def dense_inputs(case: DenseCase, max_x_rows: int | None = None):
    """Draw (w fp32 [n, k], x fp16 [m, k]) for a dense case.

    The two prefill cases share one seed: the x of the M=512 case is the first
    512 rows of the M=4096 draw, so both are drawn as [4096, k] and cut.
    """
    rng = np.random.default_rng(case.seed)
    w = weights(rng, case.n, case.k)
    m_draw = 4096 if case.name.startswith("gemm_") else case.m
    x = activations(rng, m_draw, case.k)[: case.m]
    if max_x_rows is not None:
        x = x[:max_x_rows]
    return w, x


@dataclass
class Routing:
    """Token->expert pairs sorted by (expert, token).

    pair_expert[i], pair_token[i] name pair i; offsets[e]..offsets[e+1] are the
    rows of expert e (length experts+1, offsets[0] = 0, offsets[-1] = pairs).
    """

    pair_expert: np.ndarray
    pair_token: np.ndarray
    offsets: np.ndarray
    counts: np.ndarray = field(default=None)
    choice: np.ndarray = field(default=None)   # the draws themselves: expert of (token, slot), [tokens, topk]


def route_uniform(rng: np.random.Generator, tokens: int, experts: int, topk: int) -> Routing:
    """Each token, in order, picks topk distinct experts uniformly at random."""
    choice = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])
    return _sorted_pairs(choice, experts)


def route_skewed(rng: np.random.Generator, tokens: int, experts: int, topk: int, a: float = 1.2) -> Routing:
    """Zipf-like skew: expert e has weight (e+1)^-a; topk distinct picks per token."""
    p = (np.arange(1, experts + 1, dtype=np.float64)) ** (-a)
    p /= p.sum()
    choice = np.stack([rng.choice(experts, topk, replace=False, p=p) for _ in range(tokens)])
    return _sorted_pairs(choice, experts)


def _sorted_pairs(choice: np.ndarray, experts: int) -> Routing:
    tokens, topk = choice.shape
    e = choice.reshape(-1).astype(np.int64)
    t = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.lexsort((t, e))
    e, t = e[order], t[order]
    counts = np.bincount(e, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return Routing(e.astype(np.int32), t.astype(np.int32), offsets, counts, choice.astype(np.int32))


def router_weights(rng: np.random.Generator, tokens: int, topk: int) -> np.ndarray:
    """fp32 [tokens, topk] positive weights summing to 1 per token: a softmax over
    N(0, 1) logits, standing in for a router's top-k probabilities."""
    z = rng.standard_normal((tokens, topk))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def moe_inputs(case: MoECase, experts: int | None = None):
    """Draw the MoE case: per-expert fp32 weights (list), fp16 x [tokens, k], routing.

    Expert weights are drawn one expert at a time, e = 0..E-1, so the full fp32
    bank never has to exist at once.  ``experts`` lets a caller draw only the
    first few experts' weights while keeping the routing of the full case.
    """
    rng = np.random.default_rng(case.seed)
    e_keep = case.experts if experts is None else experts
    ws = []
    for e in range(case.experts):
        w = weights(rng, case.n, case.k)
        if e < e_keep:
            ws.append(w)
    x = activations(rng, case.tokens, case.k)
    routing = route_uniform(rng, case.tokens, case.experts, case.topk)
    return ws, x, routing


def integer_activations(rng: np.random.Generator, m: int, k: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """fp16 activations holding small integers in [lo, hi] (exact-arithmetic family)."""
    return rng.integers(lo, hi + 1, size=(m, k)).astype(np.float16)


def integer_codes(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 weight codes uniform in [-8, 7] (exact-arithmetic family)."""
    return rng.integers(-8, 8, size=(n, k)).astype(np.int8)


def power_of_two_scales(rng: np.random.Generator, n: int, groups: int, lo: int = -8, hi: int = -2) -> np.ndarray:
    """fp16 scales 2^e with e uniform in [lo, hi] (exact-arithmetic family)."""
    e = rng.integers(lo, hi + 1, size=(n, groups))
    return np.ldexp(np.ones((n, groups)), e).astype(np.float16)


def code_bank(rng: np.random.Generator, experts: int, n: int, k: int) -> np.ndarray:
    """int8 weight codes [experts, n, k] uniform in [-7, 7]: the range a symmetric int4
    quantiser gives Gaussian weights (its -8 is never reached)."""
    return rng.integers(-7, 8, size=(experts, n, k), dtype=np.int8)


def scale_bank(rng: np.random.Generator, experts: int, n: int, groups: int) -> np.ndarray:
    """fp16 group scales [experts, n, groups] of the size a group of 32 N(0, 0.02^2)
    weights gets: 0.02 * U(1.5, 3.0) / 7, rounded to fp16."""
    return (WEIGHT_STD * rng.uniform(1.5, 3.0, size=(experts, n, groups)) / 7).astype(np.float16)


def moe_ffn_inputs(case: MoEFFNCase):
    """The routed-expert FFN drawn directly in quantised form (codes and scales), so both
    sides pack the same codes with their own code (quantising the 805 M Gaussian weights
    of the full bank on the host would take minutes).  Returns (gate/up codes [E, 2I, H]
    with gate rows even and up rows odd, their scales, down codes [E, H, I], their scales,
    x fp16 [T, H], routing, router weights fp32 [T, topk])."""
    rng = np.random.default_rng(case.seed)
    gu_q = code_bank(rng, case.experts, 2 * case.inter, case.hidden)
    gu_s = scale_bank(rng, case.experts, 2 * case.inter, case.hidden // case.group)
    dn_q = code_bank(rng, case.experts, case.hidden, case.inter)
    dn_s = scale_bank(rng, case.experts, case.hidden, case.inter // case.group)
    x = activations(rng, case.tokens, case.hidden)
    routing = route_uniform(rng, case.tokens, case.experts, case.topk)
    w = router_weights(rng, case.tokens, case.topk)
    return gu_q, gu_s, dn_q, dn_s, x, routing, w

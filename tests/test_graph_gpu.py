"""Decode launch chain captured in one HIP graph and replayed (the pages' CUDA-graph
decode step): every replay must leave exactly the bits of the same launches made
eagerly, with the program's own eager work and synchronisations between replays."""

import numpy as np
import pytest

import synth
from gpu_util import dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    torch_mod()
    import w4a16_int4_weight_linear_amd as w4
    return w4


def test_graph_replay_of_decode_chain_matches_eager(w4):
    torch = torch_mod()
    rng = np.random.default_rng(9100)
    # up projection (M = 1), batched decode (M = 4, MFMA kernel; M = 16, weight-streaming
    # kernel), the gated gate/up pair on both decode kernels, and a small MoE layer
    k, n = 1024, 1536
    w = synth.weights(rng, n, k)
    p, s = w4.quantize(w, 128)
    pt, st = dev(p), dev(s)
    x1 = dev(synth.activations(rng, 1, k))
    x4 = dev(synth.activations(rng, 4, k))
    x16 = dev(synth.activations(rng, 16, k))
    wm = [synth.weights(rng, 256, 512) for _ in range(6)]
    pq = [w4.quantize(a, 32) for a in wm]
    pm, sm = dev(np.stack([a for a, _ in pq])), dev(np.stack([b for _, b in pq]))
    r = synth.route_uniform(rng, 40, 6, 2)
    xm = dev(synth.activations(rng, 40, 512)[r.pair_token])
    offs = dev(r.offsets)
    y1 = torch.empty((1, n), dtype=torch.float16, device="cuda")
    y4 = torch.empty((4, n), dtype=torch.float16, device="cuda")
    y16 = torch.empty((16, n), dtype=torch.float16, device="cuda")
    g1 = torch.empty((1, n // 2), dtype=torch.float16, device="cuda")   # the n rows read as gate/up pairs
    g4 = torch.empty((4, n // 2), dtype=torch.float16, device="cuda")
    ym = torch.empty((len(r.pair_token), 256), dtype=torch.float16, device="cuda")

    def chain():
        w4.gemv(x1, pt, st, 128, out=y1)
        w4.gemv(x4, pt, st, 128, out=y4)
        w4.gemm(x16, pt, st, 128, out=y16)
        w4.gemv_swiglu(x1, pt, st, 128, out=g1)
        w4.gemv_swiglu(x4, pt, st, 128, out=g4)
        w4.grouped_gemm(xm, pm, sm, offs, 32, out=ym)

    chain()
    torch.cuda.synchronize()
    outs = (y1, y4, y16, g1, g4, ym)
    names = ("gemv m=1", "gemv m=4", "gemm m=16", "swiglu m=1", "swiglu m=4", "grouped")
    want = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()

    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: {name} differs from eager"
        chain()                              # eager launches between replays
        torch.cuda.synchronize()

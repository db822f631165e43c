"""Decode launch chain captured in one HIP graph and replayed (the pages' CUDA-graph
decode step): every replay must leave exactly the bits of the same launches made
eagerly, with the program's own eager work and synchronisations between replays,
and every replayed output must meet the fp64 oracle's bars."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, dev, host, torch_mod

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
    q_ref, s_ref = oracle.quantize(w, 128)
    p_ref = oracle.pack(q_ref)
    pt, st = dev(p), dev(s)
    x1n, x4n, x16n = (synth.activations(rng, m, k) for m in (1, 4, 16))
    x1, x4, x16 = dev(x1n), dev(x4n), dev(x16n)
    wm = [synth.weights(rng, 256, 512) for _ in range(6)]
    pq = [w4.quantize(a, 32) for a in wm]
    oq = [oracle.quantize(a, 32) for a in wm]
    pm, sm = dev(np.stack([a for a, _ in pq])), dev(np.stack([b for _, b in pq]))
    r = synth.route_uniform(rng, 40, 6, 2)
    xmn = synth.activations(rng, 40, 512)[r.pair_token]
    xm = dev(xmn)
    # the oracle's outputs of the six captured products
    refs = [oracle.linear(x1n, p_ref, s_ref, 128), oracle.linear(x4n, p_ref, s_ref, 128),
            oracle.linear(x16n, p_ref, s_ref, 128), oracle.swiglu_linear(x1n, p_ref, s_ref, 128),
            oracle.swiglu_linear(x4n, p_ref, s_ref, 128),
            oracle.grouped_linear(xmn, np.stack([oracle.pack(a) for a, _ in oq]), np.stack([b for _, b in oq]),
                                  r.offsets, 32)]
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
        for name, a, b, ref in zip(names, outs, want, refs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: {name} differs from eager"
            assert_close(host(a), ref, f"replay {rep}: {name}")
        chain()                              # eager launches between replays
        torch.cuda.synchronize()


def test_graph_replay_of_moe_layer_matches_eager(w4):
    """Routing on the device, the gathered grouped product and the combine, captured
    together: the routed row order inside an expert may change between runs, the
    offsets and the combined output may not."""
    torch = torch_mod()
    rng = np.random.default_rng(9200)
    tokens, experts, topk, k, n = 96, 12, 4, 512, 256
    wm = [synth.weights(rng, n, k) for _ in range(experts)]
    pq = [w4.quantize(a, 32) for a in wm]
    oq = [oracle.quantize(a, 32) for a in wm]
    pm, sm = dev(np.stack([a for a, _ in pq])), dev(np.stack([b for _, b in pq]))
    idsn = synth.route_uniform(rng, tokens, experts, topk).choice.astype(np.int32)
    ids = dev(idsn)
    xn = synth.activations(rng, tokens, k)
    x = dev(xn)
    wtsn = synth.router_weights(rng, tokens, topk)
    wts = dev(wtsn)
    out_ref = oracle.moe_layer(xn, idsn, wtsn, np.stack([oracle.pack(a) for a, _ in oq]), np.stack([b for _, b in oq]),
                               32)
    offs_ref = oracle.moe_route(idsn, experts)[0]
    offs = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    tok = torch.empty(tokens * topk, dtype=torch.int32, device="cuda")
    prow = torch.empty((tokens, topk), dtype=torch.int32, device="cuda")
    yp = torch.empty((tokens * topk, n), dtype=torch.float16, device="cuda")
    out = torch.empty((tokens, n), dtype=torch.float16, device="cuda")

    def layer():
        st = w4._stream(None)
        rc = w4.lib.w4a16_moe_route(w4._ptr(ids), tokens, topk, experts, w4._ptr(offs), w4._ptr(tok), w4._ptr(prow), st)
        assert rc == 0
        w4.grouped_gemm_gather(x, tok, pm, sm, offs, 32, out=yp)
        w4.moe_combine(yp, prow, wts, out=out)

    layer()
    torch.cuda.synchronize()
    want_out, want_offs = out.clone(), offs.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()

    for rep in range(4):
        out.fill_(float("nan"))
        offs.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(offs, want_offs), f"replay {rep}: offsets differ from eager"
        assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), f"replay {rep}: layer output differs"
        assert np.array_equal(host(offs), offs_ref), f"replay {rep}: offsets differ from the oracle's routing"
        assert_close(host(out), out_ref, f"replay {rep}: MoE layer")
        layer()
        torch.cuda.synchronize()

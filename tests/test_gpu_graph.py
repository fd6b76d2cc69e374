"""HIP-graph capture of the decode calls: colimoe_route_forward and
colimoe_rmsnorm_route_forward enqueue kernels only (no allocation, no host
synchronisation, no memset nodes), so a caller can capture a decode step, or
a whole stack of layers, into one graph.  Every replay must give the bits of
the same calls run eagerly; replays are interleaved with eager work and host
synchronisation, and checked one by one.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.Workload(name="graph", d=6144, f=2048, E=64, k=8, T=1, n_shared=1, zipf=1.1, seed=synth.BASE_SEED + 501)
LAYERS = 4
FXP, FP32 = 3, 1


@pytest.fixture(scope="module")
def ctx():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("graph: %d layers d=%d f=%d E=%d" % (LAYERS, W.d, W.f, W.E), flush=True)
    cap = torch.cuda.Stream()
    c = MoeContext(W.d, W.f, W.E, W.k, n_layers=LAYERS, n_shared=1, max_tokens=4, stream=cap)
    for l in range(LAYERS):
        c.load_layer(l, synth.router(W, l), synth.bias(W, l), synth.expert_blobs(W, l, 0, W.E),
                     synth.shared_blob(W, l))
    yield c, cap
    c.close()


def _step(c, x0, r, xn, idx, wts, U, flags, T):
    """Layer 0 on x0 (residual r), then layers 1.. as RMSNorm + route + forward."""
    import int4_routed_expert_fp32_amd as cm
    cm.colimoe_route_forward(c.ctx, 0, x0.data_ptr(), T, idx[0].data_ptr(), wts[0].data_ptr(), U[0].abi(),
                             r.data_ptr(), flags)
    for l in range(1, LAYERS):
        cm.colimoe_rmsnorm_route_forward(c.ctx, l, r.data_ptr(), T, 1e-6, xn.data_ptr(), idx[l].data_ptr(),
                                         wts[l].data_ptr(), U[l].abi(), flags)


@pytest.mark.parametrize("flags,T,top_p", [(FXP, 1, 1.0), (FP32, 1, 1.0), (FXP, 3, 1.0), (FXP, 1, 0.7)],
                         ids=["fxp-T1", "fp32-T1", "fxp-T3", "fxp-T1-top-p-0.7"])
def test_graph_replays_match_eager(ctx, flags, T, top_p):
    c, cap = ctx
    c.set_expert_top_p(top_p)
    try:
        _replays_match_eager(c, cap, W, flags, T)
    finally:
        c.set_expert_top_p(1.0)


# int8 experts: the one-token int8 kernels (combine in the down kernel)
W8 = synth.Workload(name="graph8", d=1024, f=512, E=32, k=4, T=1, n_shared=1, zipf=1.1, bits=8,
                    seed=synth.BASE_SEED + 502)


def test_graph_replays_match_eager_int8():
    import int4_routed_expert_fp32_amd as cm
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("graph int8: %d layers d=%d f=%d E=%d" % (LAYERS, W8.d, W8.f, W8.E), flush=True)
    cap = torch.cuda.Stream()
    c = MoeContext(W8.d, W8.f, W8.E, W8.k, n_layers=LAYERS, n_shared=1, max_tokens=1, stream=cap,
                   cfg_flags=cm.COLIMOE_CFG_INT8)
    try:
        for l in range(LAYERS):
            c.load_layer(l, synth.router(W8, l), synth.bias(W8, l), synth.expert_blobs(W8, l, 0, W8.E),
                         synth.shared_blob(W8, l))
        _replays_match_eager(c, cap, W8, 0, 1)
    finally:
        c.close()


def _replays_match_eager(c, cap, W, flags, T):
    X = torch.from_numpy(synth.activations(W.with_(T=T), stream=7 + T)).cuda()
    r = X.clone()
    xn = torch.empty_like(X)
    idx = torch.empty((LAYERS, T, W.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((LAYERS, T, W.k), dtype=torch.float32, device="cuda")
    U = [c.new_union(T) for _ in range(LAYERS)]
    torch.cuda.synchronize()
    # eager reference
    with torch.cuda.stream(cap):
        _step(c, X, r, xn, idx, wts, U, flags, T)
    c.sync()
    ref = [t.clone() for t in (r, xn, idx, wts)]
    # capture (the residual is reset before every replay, outside the graph)
    g = torch.cuda.CUDAGraph()
    r.copy_(X)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        _step(c, X, r, xn, idx, wts, U, flags, T)
    torch.cuda.synchronize()
    for rep in range(4):
        r.copy_(X)
        xn.zero_()
        idx.fill_(-1)
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        got = (r, xn, idx, wts)
        for a, b, name in zip(ref, got, ("residual", "x", "idx", "w")):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), \
                "replay %d: %s differs from the eager call" % (rep, name)
        # eager work between replays
        with torch.cuda.stream(cap):
            tmp = X.clone()
            _step(c, X, tmp, torch.empty_like(X), torch.empty_like(idx), torch.empty_like(wts),
                  [c.new_union(T) for _ in range(LAYERS)], flags, T)
        c.sync()
    print("graph %s T=%d: 4 replays bit-identical" % (W.name, T))

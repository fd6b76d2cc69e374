"""Two contexts on two streams at once: a context holds all of its state (the
workspace, the loaded layers, the union lists), so calls that overlap on the
GPU through different contexts give the bits each context gives alone.  The
two contexts hold different layers and run different token streams, one on
the fixed-point path and one on the fp32 path.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WA = synth.Workload(name="streamsA", d=2048, f=2048, E=32, k=4, T=1, n_shared=1, zipf=1.1, seed=synth.BASE_SEED + 601)
WB = synth.Workload(name="streamsB", d=2048, f=2048, E=32, k=4, T=1, n_shared=1, zipf=1.1, seed=synth.BASE_SEED + 602)
CALLS = 24
FXP, FP32 = 3, 1


def _ctx(w, stream):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    c = MoeContext(w.d, w.f, w.E, w.k, n_layers=2, n_shared=w.n_shared, max_tokens=1, stream=stream)
    for l in range(2):
        c.load_layer(l, synth.router(w, l), synth.bias(w, l), synth.expert_blobs(w, l, 0, w.E), synth.shared_blob(w, l))
    return c


def _calls(c, X, flags, interleave=None):
    """CALLS one-token route_forward calls on alternating layers; residual is
    carried from call to call.  interleave(i) runs between calls."""
    import int4_routed_expert_fp32_amd as cm
    with torch.cuda.stream(c.stream):  # every buffer made on the context's own stream
        r = X[0:1].clone()
        idx = torch.empty((CALLS, c.k), dtype=torch.int32, device="cuda")
        w = torch.empty((CALLS, c.k), dtype=torch.float32, device="cuda")
        outs = torch.empty((CALLS, X.shape[1]), dtype=torch.float32, device="cuda")
    for i in range(CALLS):
        with torch.cuda.stream(c.stream):
            x = X[i:i + 1]
            cm.colimoe_route_forward(c.ctx, i % 2, x.data_ptr(), 1, idx[i].data_ptr(), w[i].data_ptr(), None,
                                     r.data_ptr(), flags)
            outs[i].copy_(r[0])
        if interleave:
            interleave(i)
    return outs, idx, w


def test_two_contexts_two_streams():
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    print("streams: two contexts d=%d f=%d E=%d, %d calls each" % (WA.d, WA.f, WA.E, CALLS), flush=True)
    ca, cb = _ctx(WA, sa), _ctx(WB, sb)
    try:
        XA = torch.from_numpy(synth.activations(WA.with_(T=CALLS), stream=61)).cuda()
        XB = torch.from_numpy(synth.activations(WB.with_(T=CALLS), stream=62)).cuda()
        torch.cuda.synchronize()
        # each context alone
        ref_a = _calls(ca, XA, FXP)
        torch.cuda.synchronize()
        ref_b = _calls(cb, XB, FP32)
        torch.cuda.synchronize()
        # both at once: B's calls enqueued between A's, no synchronisation
        got_b = {}

        def run_b(i):
            import int4_routed_expert_fp32_amd as cm
            with torch.cuda.stream(sb):
                if i == 0:
                    got_b["r"] = XB[0:1].clone()
                    got_b["idx"] = torch.empty((CALLS, cb.k), dtype=torch.int32, device="cuda")
                    got_b["w"] = torch.empty((CALLS, cb.k), dtype=torch.float32, device="cuda")
                    got_b["outs"] = torch.empty((CALLS, XB.shape[1]), dtype=torch.float32, device="cuda")
                cm.colimoe_route_forward(cb.ctx, i % 2, XB[i:i + 1].data_ptr(), 1, got_b["idx"][i].data_ptr(),
                                         got_b["w"][i].data_ptr(), None, got_b["r"].data_ptr(), FP32)
                got_b["outs"][i].copy_(got_b["r"][0])

        got_a = _calls(ca, XA, FXP, interleave=run_b)
        torch.cuda.synchronize()
        for ref, got, name in ((ref_a, got_a, "A"), (ref_b, (got_b["outs"], got_b["idx"], got_b["w"]), "B")):
            for a, b in zip(ref, got):
                a, b = a.cpu().numpy(), b.cpu().numpy()
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "context %s differs when overlapped" % name
    finally:
        ca.close()
        cb.close()

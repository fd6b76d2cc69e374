"""One-token routing ([A] §1: 8 of the 256 experts; exact ties to the lower
index): the top-k must be taken from the final logits of this call, never
from a value left by an earlier call or by another layer.

Every call here changes x and alternates between two layers, so a selection
that read even one stale logit would disagree with the top-k of the logits
the same call returns.  Three hundred calls through colimoe_route (logits
returned) check the selection against the host's top-k of those logits id
for id, the gate weights against the softmax over them and the union lists
against the selection; route_forward of the same inputs must then select
the same experts with the same weights, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.Workload(name="route1", d=1024, f=128, E=256, k=8, T=1, n_shared=1, seed=synth.BASE_SEED + 311)
CALLS = 300


@pytest.fixture(scope="module")
def ctx():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    oracle.build(force=False)
    synth.build(force=False)
    print("route1: context d=%d E=%d k=%d, %d calls" % (W.d, W.E, W.k, CALLS), flush=True)
    c = MoeContext(W.d, W.f, W.E, W.k, n_layers=2, n_shared=W.n_shared, max_tokens=1)
    for layer in range(2):
        c.load_layer(layer, synth.router(W, layer), synth.bias(W, layer), synth.expert_blobs(W, layer, 0, W.E),
                     synth.shared_blob(W, layer))
    yield c
    c.close()


def _host_topk(l, k):
    order = np.lexsort((np.arange(l.size), -l.astype(np.float64)))
    return order[:k].astype(np.int32)


def test_selection_reads_this_calls_logits(ctx):
    X = synth.activations(W.with_(T=CALLS), stream=5)
    xs = torch.from_numpy(X).cuda()
    bad = 0
    for i in range(CALLS):
        layer = i % 2
        U = ctx.new_union(1)
        idx, w, lg = ctx.route(layer, xs[i:i + 1].contiguous(), U, want_logits=True)
        ctx.sync()
        l = lg.cpu().numpy()[0]
        g = idx.cpu().numpy()[0]
        ref = _host_topk(l, W.k)
        if not np.array_equal(g, ref):
            bad += 1
            print("call %d: gpu %s host %s" % (i, g.tolist(), ref.tolist()))
            continue
        sel = l[ref].astype(np.float64)
        wref = np.exp(sel - sel[0]) / np.exp(sel - sel[0]).sum()
        assert np.allclose(w.cpu().numpy()[0], wref, rtol=1e-5, atol=1e-7), i
        u = U.to_host()
        assert u["n_unique"] == W.k and np.array_equal(u["ids"][:W.k], np.sort(ref)), i
    assert bad == 0, "%d of %d selections differ from the top-k of their own logits" % (bad, CALLS)


def test_call_forms_select_alike(ctx):
    X = synth.activations(W.with_(T=64), stream=6)
    xs = torch.from_numpy(X).cuda()
    for i in range(64):
        x1 = xs[i:i + 1].contiguous()
        idx_a, w_a, _ = ctx.route(0, x1, ctx.new_union(1))
        res = x1.clone()
        idx_b, w_b = ctx.route_forward(0, x1, ctx.new_union(1), res)
        ctx.sync()
        assert np.array_equal(idx_a.cpu().numpy(), idx_b.cpu().numpy()), i
        assert np.array_equal(w_a.cpu().numpy().view(np.uint32), w_b.cpu().numpy().view(np.uint32)), i

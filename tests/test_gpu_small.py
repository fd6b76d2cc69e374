"""Small layers (d and f below 2048: the narrow kernels, LPR lanes per row)
through the one-call entry point (route_forward) of a one-token call: its
results must be the bits of route + forward of the same token and of the
token's row in a batched call, and within the fp32 bound of the oracle ([A]
§1-§2: 8-of-256 routing and the expert FFN, here at small sizes), at top-k
and top-p.  Rows of 33 to 63 chunks (1024 < K < 2048) take 64 lanes per row:
with 32 lanes the chunks from 32 on were dropped.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"].with_(T=6)
RAGGED = synth.Workload(name="small_ragged", d=320, f=192, E=37, k=3, T=5, n_shared=1, zipf=1.1, rho=0.3,
                        seed=synth.BASE_SEED + 701)
# 64 experts, 15 routed + shared slots, d one chunk below the wide kernels
# and f = 38 chunks: both projections at 64 lanes per row
EDGE = synth.Workload(name="small_edge", d=1984, f=1216, E=64, k=15, T=3, n_shared=1, zipf=1.1,
                      seed=synth.BASE_SEED + 702)


@pytest.fixture(scope="module", autouse=True)
def _builds():
    oracle.build(force=False)
    synth.build(force=False)


def _ctx(w):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, flush=True)
    c = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=w.T)
    P.load_layer(c, w, 0)
    return c


def _bits(a):
    return np.asarray(a).view(np.uint32)


@pytest.mark.parametrize("w", [TINY, RAGGED, EDGE], ids=lambda w: w.name)
@pytest.mark.parametrize("top_p", [1.0, 0.7], ids=["top-k", "top-p-0.7"])
def test_small_layer_one_call(w, top_p):
    ctx = _ctx(w)
    try:
        ctx.set_expert_top_p(top_p)
        ora = P.OracleLayer(w, 0)
        X = synth.activations(w, stream=71)
        worst = 0.0
        if top_p == 1.0:
            batch = P.layer_parity(ctx, w, 0, X, ora)  # T tokens: the general kernels
        for t in range(w.T):
            x1 = X[t:t + 1]
            if top_p == 1.0:
                a = P.layer_parity(ctx, w, 0, x1, ora, one_call=True)  # route_forward
                b = P.layer_parity(ctx, w, 0, x1, ora)  # route, then forward
                worst = max(worst, a["ratio"])
                assert np.array_equal(a["idx"], batch["idx"][t:t + 1]), t
                assert np.array_equal(_bits(a["out"][0]), _bits(batch["out"][t])), t
            else:
                import int4_routed_expert_fp32_amd as cm
                xt = torch.from_numpy(np.ascontiguousarray(x1)).cuda()
                outs = []
                for one in (True, False):
                    U = ctx.new_union(1)
                    res = xt.clone()
                    if one:
                        idx, wts = ctx.route_forward(0, xt, U, res, 0)
                    else:
                        idx, wts, _ = ctx.route(0, xt, U)
                        ctx.forward(0, xt, idx, wts, U, res, 0)
                    ctx.sync()
                    outs.append((idx.cpu().numpy(), wts.cpu().numpy(), res.cpu().numpy(), U.to_host()))
                a, b = outs
                b = dict(idx=b[0], w=b[1], out=b[2], union=b[3])
                a = dict(idx=a[0], w=a[1], out=a[2], union=a[3])
                assert (a["idx"] == -1).sum() == (b["idx"] == -1).sum()
            assert np.array_equal(a["idx"], b["idx"]), t
            assert np.array_equal(_bits(a["w"]), _bits(b["w"])), t
            assert np.array_equal(_bits(a["out"]), _bits(b["out"])), t
            for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
                assert np.array_equal(a["union"][key], b["union"][key]), (t, key)
        print("%s top_p %.1f: %d tokens bit-identical to route + forward, worst ratio %.3g" % (
            w.name, top_p, w.T, worst))
    finally:
        ctx.set_expert_top_p(1.0)
        ctx.close()

"""int8 gs64 expert container (COLIMOE_CFG_INT8): one-token and batched
calls against the oracle reading the same int8 blobs.  Bound per output: the
fp32 path's |gpu - oracle| <= 1e-3 (1 + |oracle|); routing, gate weights and
union lists as on the int4 path; a batched token carries the bits of the
token alone.  Paths the int8 container does not serve are refused.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TINY8 = synth.WORKLOADS["tiny"].with_(name="tiny8", bits=8, T=4)
DEC8 = synth.Workload(name="dec8", d=6144, f=2048, E=32, k=8, T=3, n_shared=1, zipf=1.1, bits=8,
                      seed=synth.BASE_SEED + 401)
RAGGED8 = synth.Workload(name="ragged8", d=320, f=192, E=37, k=3, T=3, n_shared=1, bits=8,
                         seed=synth.BASE_SEED + 402)
# beyond the one-token kernels that fuse the combine (d > 8192, f > 2048): the
# one-token calls take the general one-token kernels and the combine kernel
WIDE8 = synth.Workload(name="wide8", d=8256, f=2112, E=5, k=2, T=3, n_shared=1, bits=8,
                       seed=synth.BASE_SEED + 404)


def _ctx(w, max_tokens=4):
    import int4_routed_expert_fp32_amd as cm
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, "int8", flush=True)
    return MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=max_tokens,
                      cfg_flags=cm.COLIMOE_CFG_INT8)


@pytest.fixture(scope="module", autouse=True)
def _builds():
    oracle.build(force=False)
    synth.build(force=False)


@pytest.mark.parametrize("w", [TINY8, RAGGED8, DEC8, WIDE8], ids=lambda w: w.name)
def test_int8_layer_parity(w):
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=51)
    worst = 0.0
    with oracle.container_bits(8):
        for t in range(w.T):
            x1 = X[t:t + 1]
            a = P.layer_parity(ctx, w, 0, x1, ora, one_call=True)
            b = P.layer_parity(ctx, w, 0, x1, ora)
            assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
            worst = max(worst, a["ratio"])
    print("%s: worst ratio %.3g" % (w.name, worst))
    ctx.close()


# Batched int8 calls (2-16 tokens: per pair; the tiny layer has no shared
# expert; union16's correlated positions share experts)
U8 = synth.Workload(name="u8", d=6144, f=2048, E=32, k=8, T=16, n_shared=1, zipf=1.1, rho=0.6, bits=8,
                    seed=synth.BASE_SEED + 403)


@pytest.mark.parametrize("w,T", [(TINY8, 4), (RAGGED8, 3), (U8, 6), (U8, 16), (WIDE8, 3)],
                         ids=["tiny8-4", "ragged8-3", "u8-6", "u8-16", "wide8-3"])
def test_int8_batched_parity_and_identity(w, T):
    ctx = _ctx(w, max_tokens=T)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w.with_(T=T), stream=53)
    with oracle.container_bits(8):
        r = P.layer_parity(ctx, w.with_(T=T), 0, X, ora)
        print("%s T=%d: unique experts %d, worst ratio %.3g" % (w.name, T, r["union"]["n_unique"], r["ratio"]))
        for t in range(T):
            a = P.layer_parity(ctx, w, 0, X[t:t + 1], ora, one_call=True)
            assert np.array_equal(a["idx"][0], r["idx"][t])
            assert np.array_equal(a["out"][0].view(np.uint32), r["out"][t].view(np.uint32)), t
    ctx.close()


def test_int8_refusals():
    import int4_routed_expert_fp32_amd as cm
    w = TINY8
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    x = torch.from_numpy(synth.activations(w.with_(T=2), stream=52)).cuda()
    idx = torch.zeros((2, w.k), dtype=torch.int32, device="cuda")
    idx[:, 1] = 1
    wt = torch.full((2, w.k), 0.5, dtype=torch.float32, device="cuda")
    res = x.clone()
    # a path other than the fp32 one
    for flags in (cm.COLIMOE_FWD_FXP, cm.COLIMOE_FWD_BF16_MFMA):
        assert cm.colimoe_forward(ctx.ctx, 0, x.data_ptr(), 1, idx.data_ptr(), wt.data_ptr(), None, res.data_ptr(),
                                  flags, check=False) == cm.COLIMOE_E_SHAPE
    g = torch.empty(w.f, dtype=torch.float32, device="cuda")
    y = torch.empty(w.d, dtype=torch.float32, device="cuda")
    assert cm.lib().colimoe_debug_expert(ctx.ctx, 0, 1, x.data_ptr(), g.data_ptr(), g.data_ptr(), g.data_ptr(),
                                         y.data_ptr()) == cm.COLIMOE_E_SHAPE
    ctx.sync()
    assert torch.equal(res, x)  # refused calls have no effect
    ctx.close()


@pytest.mark.parametrize("T", [3, 16])
def test_int8_topp_batched_matches_one_token(T):
    """Expert top-p 0.7 on int8 experts, 3 and 16 tokens in one call: routing,
    weights, union lists and outputs as the oracle gives them (reading the
    same int8 blobs), and every token's row = the token routed and forwarded
    alone, bit for bit (dropped slots load nothing on either path)."""
    from tests.test_gpu_topp import check_topp_batch
    w = U8.with_(T=T)
    ctx = _ctx(w, max_tokens=T)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=57)
    ctx.set_expert_top_p(0.7)
    try:
        xt = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        U = ctx.new_union(T)
        res = xt.clone()
        idx, wt = ctx.route_forward(0, xt, U, res)
        ctx.sync()
        gidx, gw, gout = idx.cpu().numpy(), wt.cpu().numpy(), res.cpu().numpy()
        with oracle.container_bits(8):
            out, _, kept = check_topp_batch(w, ora, X.astype(np.float64), gidx, gw, U.to_host(), 0.7)
        ratio = P.assert_close(gout, out, what="int8 top-p batched output")
        print("int8 top-p T=%d: kept %s, worst ratio %.3g" % (T, kept, ratio))
        assert min(kept) < w.k
        for t in range(T):
            x1 = xt[t:t + 1].contiguous()
            r1 = x1.clone()
            i1, w1 = ctx.route_forward(0, x1, ctx.new_union(1), r1)
            ctx.sync()
            assert np.array_equal(i1.cpu().numpy()[0], gidx[t]), t
            assert np.array_equal(w1.cpu().numpy()[0].view(np.uint32), gw[t].view(np.uint32)), t
            assert np.array_equal(r1.cpu().numpy()[0].view(np.uint32), gout[t].view(np.uint32)), t
    finally:
        ctx.set_expert_top_p(1.0)
        ctx.close()

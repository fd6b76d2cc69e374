"""Adaptive expert top-p, against the oracle: one-token calls, batched calls
(whose tokens must carry the bits of the same token alone) and a
prefill-shaped call on the matrix-core path.

Rule (the oracle's): of the k experts in top-k order, keep the shortest prefix
whose gate weights (softmax over the k) reach p, re-weighted by the softmax
over the kept logits; dropped slots get id -1 and weight 0 and are not read.
The GPU decides in fp32, the oracle in fp64: a token whose kept count differs
is accepted only when the prefix mass at the boundary is within 1e-5 of p, and
its outputs are then checked under the GPU's kept set.  Outputs: the fp32
bound |gpu - oracle| <= 1e-3 (1 + |oracle|); union lists exactly.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FP32, FXP = 1, 3
P_PAGES = 0.7  # the value the pages run with
DECODE = synth.WORKLOADS["decode"]


def _ctx(w, n_layers=1, max_tokens=1):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, flush=True)
    return MoeContext(w.d, w.f, w.E, w.k, n_layers=n_layers, n_shared=w.n_shared, max_tokens=max_tokens)


@pytest.fixture(scope="module")
def dec():
    oracle.build(force=False)
    synth.build(force=False)
    ctx = _ctx(DECODE)
    P.load_layer(ctx, DECODE, 0)
    yield ctx, P.OracleLayer(DECODE, 0)
    ctx.close()


def _one_call(ctx, x, flags):
    U = ctx.new_union(1)
    res = x.clone()
    idx, w = ctx.route_forward(0, x, U, res, flags)
    ctx.sync()
    return idx.cpu().numpy()[0], w.cpu().numpy()[0], U.to_host(), res.cpu().numpy()[0]


def check_topp_token(ora, x, gidx, gw, union, gout, k, p):
    """Checks one token's top-p routing, weights, union lists and output; returns the kept count."""
    l, oidx, ow = ora.route(x[None, :])
    l, oidx, ow = l[0], oidx[0], ow[0]
    m = int(np.sum(gidx >= 0))
    assert m >= 1 and np.all(gidx[:m] >= 0) and np.all(gidx[m:] == -1), gidx
    assert np.array_equal(gidx[:m], oidx[:m]), (gidx, oidx)  # a prefix of the top-k order
    _, _, mo = oracle.expert_top_p(l, oidx, ow, p)
    if m != mo:
        cum = float(np.sum(ow[:min(m, mo)]))
        assert abs(cum - p) < 1e-5, "kept %d, oracle %d, boundary mass %.9f" % (m, mo, cum)
    wref = np.zeros(k)
    wref[:m] = oracle.softmax_selected(l, gidx[:m])
    P.assert_close(gw, wref, rel=1e-4, what="top-p gate weights")
    assert np.all(gw[m:] == 0.0)
    out, _ = ora.forward(x[None, :], gidx[None, :], wref[None, :])
    P.assert_close(gout[None, :], out, what="top-p layer output")
    ou = oracle.union(gidx[None, :], ora.w.E)
    assert union["n_unique"] == ou["n_unique"] == m
    for key in ("ids", "offsets", "pair_of"):
        assert np.array_equal(union[key], ou[key]), key
    for key in ("pair_token", "pair_slot"):
        assert np.array_equal(union[key][:m], ou[key][:m]), key
    return m


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
def test_topp_decode_parity(dec, flags):
    ctx, ora = dec
    ctx.set_expert_top_p(P_PAGES)
    try:
        X = synth.activations(DECODE.with_(T=12), stream=31)
        kept = []
        for t in range(X.shape[0]):
            x = torch.from_numpy(X[t:t + 1]).cuda()
            gidx, gw, union, gout = _one_call(ctx, x, flags)
            kept.append(check_topp_token(ora, X[t].astype(np.float64), gidx, gw, union, gout, DECODE.k, P_PAGES))
            # route, then forward with the lists route wrote: the same bits
            U = ctx.new_union(1)
            idx, w, _ = ctx.route(0, x, U)
            res = x.clone()
            ctx.forward(0, x, idx, w, U, res, flags)
            ctx.sync()
            assert np.array_equal(idx.cpu().numpy()[0], gidx)
            assert np.array_equal(res.cpu().numpy()[0].view(np.uint32), gout.view(np.uint32))
        print("top-p %.2f: experts kept per token" % P_PAGES, kept, "mean %.2f of %d" % (np.mean(kept), DECODE.k))
        assert min(kept) < DECODE.k  # the workload does drop experts
    finally:
        ctx.set_expert_top_p(1.0)


def test_topp_one_is_plain_topk(dec):
    ctx, ora = dec
    x = torch.from_numpy(synth.activations(DECODE.with_(T=1), stream=32)).cuda()
    a = _one_call(ctx, x, FXP)
    ctx.set_expert_top_p(0.5)
    ctx.set_expert_top_p(1.0)
    b = _one_call(ctx, x, FXP)
    assert np.array_equal(a[0], b[0]) and np.all(a[0] >= 0)
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))


def test_topp_stack_step_matches_two_calls(dec):
    """colimoe_rmsnorm_route_forward with top-p: the bits of colimoe_rmsnorm
    followed by colimoe_route_forward."""
    ctx, ora = dec
    ctx.set_expert_top_p(P_PAGES)
    try:
        R = torch.from_numpy(synth.activations(DECODE.with_(T=3), stream=33) * 2.0).cuda()
        for t in range(3):
            r1, r2 = R[t:t + 1].clone(), R[t:t + 1].clone()
            x1, x2 = torch.empty_like(r1), torch.empty_like(r2)
            U1, U2 = ctx.new_union(1), ctx.new_union(1)
            i1, w1 = ctx.rmsnorm_route_forward(0, r1, 1e-6, x1, U1, FXP)
            ctx.rmsnorm(r2, 1e-6, x2)
            i2, w2 = ctx.route_forward(0, x2, U2, r2, FXP)
            ctx.sync()
            assert torch.equal(i1, i2) and torch.equal(x1, x2)
            assert np.array_equal(w1.cpu().numpy().view(np.uint32), w2.cpu().numpy().view(np.uint32))
            assert np.array_equal(r1.cpu().numpy().view(np.uint32), r2.cpu().numpy().view(np.uint32))
    finally:
        ctx.set_expert_top_p(1.0)


def test_topp_rejections():
    import int4_routed_expert_fp32_amd as cm
    w = synth.WORKLOADS["tiny"]
    ctx = _ctx(w, max_tokens=2)
    P.load_layer(ctx, w, 0)
    for bad in (0.0, -0.5, 1.5, math.nan):
        assert cm.colimoe_set_expert_top_p(ctx.ctx, bad, check=False) == cm.COLIMOE_E_ARG
    ctx.close()


def check_topp_batch(w, ora, X, gidx, gw, union, p):
    """Every token's kept prefix and weights (the rule of check_topp_token),
    the union lists of the whole routing against the oracle's; returns the
    oracle's outputs and L1 norms under the GPU's routing, and the kept counts."""
    L, oidx, ow = ora.route(X)
    T = X.shape[0]
    wref = np.zeros((T, w.k))
    kept = []
    for t in range(T):
        m = int(np.sum(gidx[t] >= 0))
        assert m >= 1 and np.all(gidx[t, :m] >= 0) and np.all(gidx[t, m:] == -1), gidx[t]
        assert np.array_equal(gidx[t, :m], oidx[t, :m]), (t, gidx[t], oidx[t])
        _, _, mo = oracle.expert_top_p(L[t], oidx[t], ow[t], p)
        if m != mo:
            cum = float(np.sum(ow[t, :min(m, mo)]))
            assert abs(cum - p) < 1e-5, "token %d kept %d, oracle %d, boundary mass %.9f" % (t, m, mo, cum)
        wref[t, :m] = oracle.softmax_selected(L[t], gidx[t, :m])
        kept.append(m)
    P.assert_close(gw, wref, rel=1e-4, what="top-p gate weights")
    assert np.all(gw[gidx < 0] == 0.0)
    ou = oracle.union(gidx, w.E)
    assert union["n_unique"] == ou["n_unique"]
    n = int(np.sum(gidx >= 0))
    for key in ("ids", "offsets", "pair_of"):
        assert np.array_equal(union[key], ou[key]), key
    for key in ("pair_token", "pair_slot"):
        assert np.array_equal(union[key][:n], ou[key][:n]), key
    out, l1 = ora.forward(X, gidx, wref)
    return out, l1, kept


# Batched calls with expert top-p: up to 16 tokens (top-k and lists in one
# launch; 24 pairs ranked in one wave, 128 through the per-expert lane
# masks), 40 tokens (the matrix-core router, the general top-k and union
# kernels), each on both fp32-class paths.  Every token's row of the batch
# must carry the bits of the same token forwarded alone under its routing,
# and up to 16 tokens also those of the token routed alone.
BATCH_T = [3, 16, 40]


@pytest.fixture(scope="module")
def u16():
    w = synth.WORKLOADS["union16"].with_(T=max(BATCH_T))
    ctx = _ctx(w, max_tokens=w.T)
    P.load_layer(ctx, w, 0)
    yield ctx, P.OracleLayer(w, 0), w
    ctx.close()


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
@pytest.mark.parametrize("T", BATCH_T)
def test_topp_batched_matches_one_token(u16, T, flags):
    ctx, ora, w = u16
    X = synth.activations(w, stream=36)[:T]
    ctx.set_expert_top_p(P_PAGES)
    try:
        xt = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        U = ctx.new_union(T)
        res = xt.clone()
        idx, wt = ctx.route_forward(0, xt, U, res, flags)
        ctx.sync()
        gidx, gw, gout = idx.cpu().numpy(), wt.cpu().numpy(), res.cpu().numpy()
        out, _, kept = check_topp_batch(w, ora, X.astype(np.float64), gidx, gw, U.to_host(), P_PAGES)
        ratio = P.assert_close(gout, out, what="top-p batched layer output")
        print("T=%d: experts kept per token %s (mean %.2f of %d), unique %d, worst ratio %.3g" % (
            T, kept, np.mean(kept), w.k, U.to_host()["n_unique"], ratio))
        assert min(kept) < w.k
        # forward with the lists rebuilt from idx (dropped slots are -1): the same bits
        res2 = xt.clone()
        ctx.forward(0, xt, idx, wt, None, res2, flags)
        ctx.sync()
        assert np.array_equal(res2.cpu().numpy().view(np.uint32), gout.view(np.uint32))
        for t in range(T):
            x1 = xt[t:t + 1].contiguous()
            # the token's routing row alone through colimoe_forward: the bits
            # of its row in the batch
            r1 = x1.clone()
            ctx.forward(0, x1, idx[t:t + 1].contiguous(), wt[t:t + 1].contiguous(), None, r1, flags)
            ctx.sync()
            assert np.array_equal(r1.cpu().numpy()[0].view(np.uint32), gout[t].view(np.uint32)), t
            if T <= 16:
                # up to 16 tokens the router sums every logit as one token's
                # does, so routing the token alone gives the same bits again
                U1 = ctx.new_union(1)
                r2 = x1.clone()
                i1, w1 = ctx.route_forward(0, x1, U1, r2, flags)
                ctx.sync()
                assert np.array_equal(i1.cpu().numpy()[0], gidx[t]), t
                assert np.array_equal(w1.cpu().numpy()[0].view(np.uint32), gw[t].view(np.uint32)), t
                assert np.array_equal(r2.cpu().numpy()[0].view(np.uint32), gout[t].view(np.uint32)), t
    finally:
        ctx.set_expert_top_p(1.0)


def test_topp_prefill_shape_mfma():
    """A prefill-shaped call (T k >= 64 E: the bf16 matrix-core path) with
    expert top-p: routing, weights and union lists as above, outputs within
    the bf16 bound 2e-2 N_r."""
    w = synth.Workload(name="mfma_a", d=384, f=256, E=24, k=4, T=400, n_shared=1, zipf=1.1,
                       seed=synth.BASE_SEED + 201)
    ctx = _ctx(w, max_tokens=w.T)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    ctx.set_expert_top_p(P_PAGES)
    X = synth.activations(w, stream=37)
    xt = torch.from_numpy(X).cuda()
    U = ctx.new_union(w.T)
    res = xt.clone()
    idx, wt = ctx.route_forward(0, xt, U, res, 2)
    ctx.sync()
    gidx, gw, gout = idx.cpu().numpy(), wt.cpu().numpy(), res.cpu().numpy()
    out, l1, kept = check_topp_batch(w, ora, X.astype(np.float64), gidx, gw, U.to_host(), P_PAGES)
    ratio = float(np.max(np.abs(gout.astype(np.float64) - out) / (2e-2 * l1)))
    print("mfma top-p: mean kept %.2f of %d, worst bf16 ratio %.3g" % (np.mean(kept), w.k, ratio))
    assert ratio <= 1.0
    assert min(kept) < w.k
    ctx.close()


# odd shapes on the fp32 kernels: partial lane groups, E not a multiple of 64,
# with and without a shared expert
RAGGED = synth.Workload(name="ragged", d=320, f=192, E=37, k=3, T=6, n_shared=1, zipf=1.1, rho=0.3,
                        seed=synth.BASE_SEED + 101)
TINY6 = synth.WORKLOADS["tiny"].with_(T=6)


@pytest.mark.parametrize("w", [RAGGED, TINY6], ids=lambda w: w.name)
def test_topp_small_shapes(w):
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    ctx.set_expert_top_p(0.5)
    X = synth.activations(w, stream=35)
    kept = []
    for t in range(w.T):
        x = torch.from_numpy(X[t:t + 1]).cuda()
        U = ctx.new_union(1)
        res = x.clone()
        idx, wt = ctx.route_forward(0, x, U, res, FP32)
        ctx.sync()
        kept.append(check_topp_token(ora, X[t].astype(np.float64), idx.cpu().numpy()[0], wt.cpu().numpy()[0],
                                     U.to_host(), res.cpu().numpy()[0], w.k, 0.5))
    print(w.name, "experts kept per token", kept)
    ctx.close()

"""Exact ties in routing, on the GPU, through colimoe_route and
colimoe_route_forward.

The method routes deterministically: of experts whose logits are equal, the
lower index is selected first ([A] §1, 8 of 256 experts routed; [A] §4,
routing semantics are never changed silently).  Random logits never tie, so
these cases build ties on purpose:

* x = 0 (and x = -0) with no bias: every logit is a zero, all equal, so the
  selection is experts 0..k-1 in that order and every gate weight is 1/k
  (the router's sums start from +0, so its logits are never -0; the top-k
  key also folds -0 into +0, so the two would tie if they met);
* router rows copied between experts (with equal biases): their logits are
  the same fp32 value for every token, the lower index must come first, and a
  group of equal logits that straddles the k-th place keeps its lowest ids.

Each case runs through every routing form: one token, up to 16 tokens (with
and without union lists), and the many-token router.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.Workload(name="ties", d=512, f=128, E=256, k=8, T=40, n_shared=1, seed=synth.BASE_SEED + 301)
G1 = [200, 7]                                # bias +10: always the two largest logits
G2 = [250, 100, 60, 30, 31, 45, 12, 90]      # bias +5: six of the eight fill places 2..7
EXPECT = [7, 200, 12, 30, 31, 45, 60, 90]


@pytest.fixture(scope="module")
def ctx_and_layers():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    oracle.build(force=False)
    synth.build(force=False)
    print("ties: context d=%d f=%d E=%d k=%d" % (W.d, W.f, W.E, W.k), flush=True)
    ctx = MoeContext(W.d, W.f, W.E, W.k, n_layers=2, n_shared=W.n_shared, max_tokens=W.T)
    ex = synth.expert_blobs(W, 0, 0, W.E)
    sh = synth.shared_blob(W, 0)
    R0 = synth.router(W, 0)
    ctx.load_layer(0, R0, None, ex, sh)            # layer 0: plain router, no bias
    R1 = R0.copy()
    b1 = np.zeros(W.E, np.float32)
    for e in G1:
        R1[e] = R0[G1[1]]
        b1[e] = 10.0
    for e in G2:
        R1[e] = R0[G2[6]]
        b1[e] = 5.0
    ctx.load_layer(1, R1, b1, ex, sh)              # layer 1: duplicated rows
    yield ctx, {0: (R0, None), 1: (R1, b1)}, ex, sh
    ctx.close()


def _route(ctx, layer, X, form):
    """idx, w, logits (or None), union (or None) through one call form."""
    x = torch.from_numpy(np.ascontiguousarray(X, np.float32)).cuda()
    T = X.shape[0]
    if form == "route":
        U = ctx.new_union(T)
        idx, w, lg = ctx.route(layer, x, U, want_logits=True)
    elif form == "route_no_union":
        U = None
        idx, w, lg = ctx.route(layer, x, None, want_logits=False)
    else:  # route_forward
        U = ctx.new_union(T)
        res = x.clone()
        idx, w = ctx.route_forward(layer, x, U, res)
        lg = None
    ctx.sync()
    return (idx.cpu().numpy(), w.cpu().numpy(), None if lg is None else lg.cpu().numpy(),
            None if U is None else U.to_host())


FORMS = [(1, "route"), (1, "route_forward"), (1, "route_no_union"), (5, "route"), (5, "route_no_union"),
         (16, "route"), (5, "route_forward"), (40, "route"), (40, "route_no_union")]


@pytest.mark.parametrize("T,form", FORMS, ids=["T%d-%s" % f for f in FORMS])
@pytest.mark.parametrize("zero", ["+0", "-0"])
def test_all_logits_zero_select_the_first_k(ctx_and_layers, T, form, zero):
    """x = 0 and no bias: every logit is a zero; the selection is 0..k-1 and
    every gate weight is exactly 1/k (exp(0) / k)."""
    ctx, _, _, _ = ctx_and_layers
    X = np.full((T, W.d), 0.0 if zero == "+0" else -0.0, np.float32)
    idx, w, lg, union = _route(ctx, 0, X, form)
    if lg is not None:
        assert np.all(lg == 0.0), "logits of a zero input must be zeros"
        print("T=%d %s: %d of %d logits are -0" % (T, form, int(np.signbit(lg).sum()), lg.size))
    assert np.array_equal(idx, np.tile(np.arange(W.k, dtype=np.int32), (T, 1))), idx[:2]
    assert np.array_equal(w.view(np.uint32), np.full((T, W.k), np.float32(1.0 / W.k)).view(np.uint32)), w[:2]
    if union is not None:
        o = oracle.union(idx, W.E)
        assert union["n_unique"] == W.k == o["n_unique"]
        for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
            assert np.array_equal(union[key], o[key]), key


@pytest.mark.parametrize("T,form", FORMS, ids=["T%d-%s" % f for f in FORMS])
def test_duplicated_router_rows_go_to_the_lower_index(ctx_and_layers, T, form):
    """Equal logits from copied router rows: the lower index comes first,
    and a tied group cut at the k-th place keeps its lowest ids.  The oracle
    sees the same exact ties in fp64 and must agree id for id; weights,
    union lists and (route_forward) the layer output are checked as in every
    parity test."""
    ctx, layers, ex, sh = ctx_and_layers
    R1, b1 = layers[1]
    X = synth.activations(W, stream=T)[:T]
    idx, w, lg, union = _route(ctx, 1, X, form)
    L, oidx, ow = oracle.route(R1, b1, X.astype(np.float64), W.k)
    assert np.array_equal(oidx, np.tile(np.array(EXPECT, np.int32), (T, 1))), "oracle: " + str(oidx[0])
    assert np.array_equal(idx, oidx), "GPU %s vs oracle %s" % (idx[0], oidx[0])
    if lg is not None:
        for grp in (G1, G2):
            assert np.all(lg[:, grp] == lg[:, grp[:1]]), "copied rows must give equal fp32 logits"
        P.assert_close(lg, L, rel=1e-4, what="logits")
    wref = np.stack([oracle.softmax_selected(L[t], idx[t]) for t in range(T)])
    P.assert_close(w, wref, rel=1e-4, what="gate weights")
    # equal logits give equal weights, bit for bit
    assert np.all(w[:, 0] == w[:, 1]) and np.all(w[:, 2:] == w[:, 2:3])
    if union is not None:
        o = oracle.union(idx, W.E)
        assert union["n_unique"] == o["n_unique"]
        for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
            assert np.array_equal(union[key], o[key]), key
    if form == "route_forward":
        x = torch.from_numpy(np.ascontiguousarray(X, np.float32)).cuda()
        res = x.clone()
        ctx.route_forward(1, x, ctx.new_union(T), res)
        ctx.sync()
        blobs = {e: ex[e] for e in EXPECT}
        out, _ = oracle.moe_layer(X, W.d, W.f, blobs, sh, idx, wref, E=W.E)
        P.assert_close(res.cpu().numpy(), out, what="layer output")


# The same cases on a small router (E <= 32, d <= 2048): one-token calls route
# and select in one block there.
WS = synth.Workload(name="ties_small", d=512, f=128, E=24, k=4, T=1, n_shared=1, seed=synth.BASE_SEED + 302)
G1S = [20, 3]            # bias +10: the two largest logits
G2S = [22, 10, 5, 6, 15]  # bias +5: the tied group cut at the 4th place keeps 5 and 6
EXPECT_S = [3, 20, 5, 6]
FORMS_S = ["route", "route_forward", "route_no_union"]


@pytest.fixture(scope="module")
def small_ctx():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    oracle.build(force=False)
    synth.build(force=False)
    print("ties: context d=%d f=%d E=%d k=%d" % (WS.d, WS.f, WS.E, WS.k), flush=True)
    ctx = MoeContext(WS.d, WS.f, WS.E, WS.k, n_layers=2, n_shared=WS.n_shared, max_tokens=1)
    ex = synth.expert_blobs(WS, 0, 0, WS.E)
    sh = synth.shared_blob(WS, 0)
    R0 = synth.router(WS, 0)
    ctx.load_layer(0, R0, None, ex, sh)
    R1 = R0.copy()
    b1 = np.zeros(WS.E, np.float32)
    for e in G1S:
        R1[e] = R0[G1S[1]]
        b1[e] = 10.0
    for e in G2S:
        R1[e] = R0[G2S[3]]
        b1[e] = 5.0
    ctx.load_layer(1, R1, b1, ex, sh)
    yield ctx, R1, b1, ex, sh
    ctx.close()


@pytest.mark.parametrize("form", FORMS_S)
@pytest.mark.parametrize("zero", ["+0", "-0"])
def test_small_router_zero_logits(small_ctx, form, zero):
    ctx = small_ctx[0]
    X = np.full((1, WS.d), 0.0 if zero == "+0" else -0.0, np.float32)
    idx, w, lg, union = _route(ctx, 0, X, form)
    if lg is not None:
        assert np.all(lg == 0.0)
    assert np.array_equal(idx, np.arange(WS.k, dtype=np.int32)[None, :]), idx
    assert np.array_equal(w.view(np.uint32), np.full((1, WS.k), np.float32(1.0 / WS.k)).view(np.uint32)), w
    if union is not None:
        o = oracle.union(idx, WS.E)
        for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
            assert np.array_equal(union[key], o[key]), key


@pytest.mark.parametrize("form", FORMS_S)
def test_small_router_duplicated_rows(small_ctx, form):
    ctx, R1, b1, ex, sh = small_ctx
    X = synth.activations(WS, stream=5)[:1]
    idx, w, lg, union = _route(ctx, 1, X, form)
    L, oidx, ow = oracle.route(R1, b1, X.astype(np.float64), WS.k)
    assert np.array_equal(oidx[0], np.array(EXPECT_S, np.int32)), "oracle: " + str(oidx[0])
    assert np.array_equal(idx, oidx), "GPU %s vs oracle %s" % (idx[0], oidx[0])
    if lg is not None:
        for grp in (G1S, G2S):
            assert np.all(lg[:, grp] == lg[:, grp[:1]])
        P.assert_close(lg, L, rel=1e-4, what="logits")
    wref = np.stack([oracle.softmax_selected(L[0], idx[0])])
    P.assert_close(w, wref, rel=1e-4, what="gate weights")
    assert w[0, 0] == w[0, 1] and np.all(w[0, 2:] == w[0, 2])
    if union is not None:
        o = oracle.union(idx, WS.E)
        for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
            assert np.array_equal(union[key], o[key]), key

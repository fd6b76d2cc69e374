"""Helpers shared by the GPU parity tests: loading synthetic layers, running the
oracle on the tokens a test checks, and the acceptance rules.

Acceptance (per output o of the fp32 path):  |gpu - oracle| <= 1e-3 * (1 + |oracle|).
Routing: the GPU's expert ids must equal the oracle's, except for a token whose
k-th and (k+1)-th fp64 logits differ by less than 1e-5 (several routings are
then correct); adjacent selected experts closer than 1e-5 may swap order.  A
token routed differently is checked against the oracle re-run on the GPU's ids.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

FP32_REL = 1e-3
TIE_TAU = 1e-5


def load_layer(ctx, w: synth.Workload, layer: int, seed_layer: int = None):
    """Generate layer `seed_layer` (default: layer) of workload w and load it as `layer`."""
    sl = layer if seed_layer is None else seed_layer
    R = synth.router(w, sl)
    b = synth.bias(w, sl)
    ex = synth.expert_blobs(w, sl, 0, w.E)
    sh = synth.shared_blob(w, sl)
    ctx.load_layer(layer, R, b, ex, sh)
    return R, b


def check_routing(L: np.ndarray, gidx: np.ndarray, k: int, tau: float = TIE_TAU):
    """Returns (n_exact, tokens routed differently but validly).  Raises AssertionError otherwise."""
    T, E = L.shape
    differ = []
    for t in range(T):
        l = L[t]
        order = np.lexsort((np.arange(E), -l))
        ref = order[:k]
        g = np.asarray(gidx[t], dtype=np.int64)
        if np.array_equal(g, ref):
            continue
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < E, (t, g)
        lk = l[ref[-1]]
        gap = lk - l[order[k]] if k < E else np.inf
        in_g = np.zeros(E, dtype=bool)
        in_g[g] = True
        if set(g.tolist()) != set(ref.tolist()):
            assert gap < tau, "token %d: routed set differs with a clear boundary gap %g" % (t, gap)
            assert np.all(l[g] >= lk - tau) and np.all(l[~in_g] <= lk + tau), (t, g, ref)
            differ.append(t)
        # order among the selected: non-increasing up to tau
        assert np.all(l[g[:-1]] >= l[g[1:]] - tau), ("order", t, g, l[g])
    return T - len(differ), differ


def assert_close(gpu: np.ndarray, ora: np.ndarray, rel: float = FP32_REL, what: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), what + ": non-finite GPU output"
    err = np.abs(gpu - ora)
    bound = rel * (1.0 + np.abs(ora))
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, "%s: max |gpu-oracle|/bound = %.3g at %s (gpu %r, oracle %r)" % (
        what, ratio.max(), worst, gpu[worst], ora[worst])
    return float(ratio.max())


class OracleLayer:
    """Oracle view of one synthetic layer; generates only the experts it needs."""

    def __init__(self, w: synth.Workload, layer: int):
        self.w, self.layer = w, layer
        self.R = synth.router(w, layer)
        self.b = synth.bias(w, layer)
        self.shared = synth.shared_blob(w, layer)
        self._blobs = {}

    def blobs(self, ids):
        """Blobs of the experts in ids (an id of -1, a slot dropped by expert top-p, needs none)."""
        ids = [int(e) for e in ids if int(e) >= 0]
        need = sorted(set(ids) - set(self._blobs))
        for e in need:
            self._blobs[e] = synth.expert_blobs(self.w, self.layer, e, e + 1)[0].copy()
        return {e: self._blobs[e] for e in set(ids)}

    def route(self, X):
        return oracle.route(self.R, self.b, np.asarray(X, dtype=np.float64), self.w.k)

    def forward(self, X, idx, wts, residual=None):
        X = np.atleast_2d(np.asarray(X, dtype=np.float64))
        ex = self.blobs(np.asarray(idx).ravel())
        return oracle.moe_layer(X, self.w.d, self.w.f, ex, self.shared, idx, wts, residual, E=self.w.E)

    def weights_for(self, L_row, idx_row):
        return oracle.softmax_selected(L_row, np.asarray(idx_row, dtype=np.int32))


def layer_parity(ctx, w: synth.Workload, layer: int, X: np.ndarray, ora: OracleLayer, residual=None, flags=0,
                 one_call=False):
    """Route + forward on the GPU (or colimoe_route_forward if one_call), then
    check routing, weights and outputs against the oracle.

    Returns dict with the GPU results and the worst error ratio."""
    import torch
    dev = ctx.device
    xt = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev)
    T = X.shape[0]
    U = ctx.new_union(T)
    res = xt.clone() if residual is None else torch.from_numpy(np.ascontiguousarray(residual, np.float32)).to(dev)
    if one_call:
        idx, wts = ctx.route_forward(layer, xt, U, res, flags)
        glog = None
    else:
        idx, wts, logits = ctx.route(layer, xt, U, want_logits=True)
        ctx.forward(layer, xt, idx, wts, U, res, flags)
    ctx.sync()
    gidx = idx.cpu().numpy()
    gw = wts.cpu().numpy()
    gout = res.cpu().numpy()
    L, oidx, ow = ora.route(X)
    if not one_call:
        # logits: fp32 dot of d terms vs fp64
        assert_close(logits.cpu().numpy(), L, rel=1e-4, what="logits")
    n_exact, differ = check_routing(L, gidx, w.k)
    # weights for the GPU's selection vs the oracle's softmax over the same selection
    wref = np.stack([ora.weights_for(L[t], gidx[t]) for t in range(T)])
    assert_close(gw, wref, rel=1e-4, what="gate weights")
    # outputs: the oracle under the GPU's routing (identical to its own where the sets agree)
    out, l1 = ora.forward(X, gidx, wref, residual)
    ratio = assert_close(gout, out, what="layer output")
    # the union lists of the GPU's routing, exactly as the oracle builds them
    union = U.to_host()
    ou = oracle.union(gidx, w.E)
    assert union["n_unique"] == ou["n_unique"], "union: unique count"
    for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
        assert np.array_equal(union[key], ou[key]), "union list " + key
    return dict(idx=gidx, w=gw, out=gout, ratio=ratio, differ=differ, union=union, oracle_out=out)

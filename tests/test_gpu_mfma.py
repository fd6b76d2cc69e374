"""GPU parity of the bf16 MFMA path (prefill-shaped calls) against the CPU oracle.

Bound per output r: |gpu - oracle| <= 2e-2 * N_r, where N_r is the oracle's L1
norm of the products that make up output r (|residual_r| + sum_j |w_j| *
sum_c |Wd_j[r][c] h_j[c]| + the shared expert's terms).  Routing ids and union
lists follow the same rules as the fp32 path: exact, except on near-ties.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_REL = 2e-2
MFMA = 2
PREFILL = synth.WORKLOADS["prefill2048"]
# several M-blocks per expert (Zipf bias: some experts over 128 rows), M-tiles
# with a ragged last row count, K = 6 and 4 groups
MFMA_A = synth.Workload(name="mfma_a", d=384, f=256, E=24, k=4, T=400, n_shared=1, zipf=1.1,
                        seed=synth.BASE_SEED + 201)
# d = 320: the last 128-row tile of the down product is half empty; f = 192
MFMA_B = synth.Workload(name="mfma_b", d=320, f=192, E=37, k=3, T=200, n_shared=1, zipf=1.1, rho=0.3,
                        seed=synth.BASE_SEED + 202)
# a few tokens: every M-block has a single partial M-tile; no shared expert
MFMA_C = synth.Workload(name="mfma_c", d=256, f=128, E=16, k=2, T=5, n_shared=0, seed=synth.BASE_SEED + 203)


def _ctx(w, max_tokens=None):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, w.T, flush=True)
    return MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=max_tokens or w.T)


@pytest.fixture(scope="module", autouse=True)
def _builds():
    oracle.build(force=False)
    synth.build(force=False)


def assert_bf16_bound(gpu, ora, l1, what):
    gpu = np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(gpu)), what + ": non-finite GPU output"
    err = np.abs(gpu - ora)
    ratio = err / (BF16_REL * l1)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, "%s: max |gpu-oracle|/(2e-2 N) = %.3g at %s" % (what, ratio.max(), worst)
    return float(ratio.max())


def run_layer(ctx, w, X, flags):
    dev = ctx.device
    xt = torch.from_numpy(np.ascontiguousarray(X, np.float32)).to(dev)
    U = ctx.new_union(X.shape[0])
    idx, wts, logits = ctx.route(0, xt, U, want_logits=True)
    res = xt.clone()
    ctx.forward(0, xt, idx, wts, U, res, flags)
    ctx.sync()
    return idx.cpu().numpy(), wts.cpu().numpy(), logits.cpu().numpy(), res.cpu().numpy(), U.to_host()


def check_route_and_union(w, ora, X, gidx, gw, glog, union):
    L, _, _ = ora.route(X)
    P.assert_close(glog, L, rel=1e-4, what="logits")
    _, differ = P.check_routing(L, gidx, w.k)
    o = oracle.union(gidx, w.E)
    assert union["n_unique"] == o["n_unique"]
    for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
        assert np.array_equal(union[key], o[key]), key
    return L, differ


@pytest.mark.parametrize("w", [MFMA_A, MFMA_B, MFMA_C], ids=lambda w: w.name)
def test_mfma_layer_parity_small(w):
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    gidx, gw, glog, gout, union = run_layer(ctx, w, X, MFMA)
    L, differ = check_route_and_union(w, ora, X, gidx, gw, glog, union)
    wref = np.stack([ora.weights_for(L[t], gidx[t]) for t in range(w.T)])
    P.assert_close(gw, wref, rel=1e-4, what="gate weights")
    out, l1 = ora.forward(X, gidx, wref)
    ratio = assert_bf16_bound(gout, out, l1, w.name)
    counts = np.diff(union["offsets"])
    print("%s: worst ratio %.3g, near-tie tokens %s, rows per expert max %d" % (w.name, ratio, differ, counts.max()))


def test_mfma_is_auto_for_prefill_shapes():
    """T*k >= 64*E selects the MFMA path: AUTO and the forced flag give the same bits."""
    w = MFMA_A
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    X = synth.activations(w, stream=3)
    assert w.T * w.k >= 64 * w.E
    a = run_layer(ctx, w, X, 0)[3]
    b = run_layer(ctx, w, X, MFMA)[3]
    c = run_layer(ctx, w, X, 1)[3]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert not np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_prefill2048_parity():
    """Full-size prefill call: all 2048 routings and the union lists are
    checked exactly, and every output of every token against the oracle
    under the bf16 bound (the oracle's grouped form: each expert dequantised
    once, fp64 products over all its tokens)."""
    import time
    w = PREFILL
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    gidx, gw, glog, gout, union = run_layer(ctx, w, X, 0)  # AUTO: T*k = 64*E
    ctx.close()
    L, differ = check_route_and_union(w, ora, X, gidx, gw, glog, union)
    wref = np.stack([ora.weights_for(L[t], gidx[t]) for t in range(w.T)])
    P.assert_close(gw, wref, rel=1e-4, what="gate weights")
    t0 = time.time()
    out, l1 = oracle.moe_layer_grouped(X, w.d, w.f, lambda e: synth.expert_blobs(w, 0, e, e + 1)[0], ora.shared,
                                       gidx, wref)
    ratio = assert_bf16_bound(gout, out, l1, "prefill2048")
    counts = np.diff(union["offsets"])
    print("prefill2048: %d unique experts, rows per expert max %d, >=64: %d; worst ratio %.3g over all %d tokens "
          "(oracle %.1f s); near-tie tokens %d" % (union["n_unique"], counts.max(), int((counts >= 64).sum()), ratio,
                                                  w.T, time.time() - t0, len(differ)))


def test_mfma_block_class_boundaries():
    """A forced routing that gives experts 1, 32, 33, 128, 129, 160, 256, 257,
    288 and 289 rows: M-blocks at both edges of the one-M-tile class (<= 32
    rows), of the 256-row blocks (a 257-row expert leaves a one-row block, a
    288-row one a 32-row block, a 289-row one a 33-row block), and blocks of
    every M-tile count from 2 to 8, through the bf16 path, against the oracle
    under the same routing."""
    w = synth.Workload(name="mfma_edges", d=384, f=256, E=24, k=4, T=512, n_shared=1, seed=synth.BASE_SEED + 204)
    counts = {0: 32, 1: 33, 2: 128, 3: 129, 4: 160, 5: 1, 6: 257, 7: 256, 8: 288, 9: 289, 10: 70, 11: 200}
    rest = w.T * w.k - sum(counts.values())
    others = list(range(12, w.E))
    for i, e in enumerate(others):
        counts[e] = rest // len(others) + (1 if i < rest % len(others) else 0)
    pairs = [e for e in sorted(counts) for _ in range(counts[e])]
    # pair i goes to token i mod T: an expert's pairs land on distinct tokens
    idx = np.zeros((w.T, w.k), dtype=np.int32)
    fill = np.zeros(w.T, dtype=np.int64)
    for i, e in enumerate(pairs):
        t = i % w.T
        idx[t, fill[t]] = e
        fill[t] += 1
    assert np.all(fill == w.k) and all(len(set(r)) == w.k for r in idx.tolist())
    rng = np.random.default_rng(204)
    wts = rng.uniform(0.05, 1.0, size=(w.T, w.k))
    wts = (wts / wts.sum(axis=1, keepdims=True)).astype(np.float32)
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    X = synth.activations(w, stream=9)
    xt = torch.from_numpy(X).cuda()
    res = xt.clone()
    ctx.forward(0, xt, torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda(), None, res, MFMA)
    ctx.sync()
    ora = P.OracleLayer(w, 0)
    out, l1 = ora.forward(X, idx, wts.astype(np.float64))
    r = assert_bf16_bound(res.cpu().numpy(), out, l1, w.name)
    print("%s: worst ratio %.3g" % (w.name, r))

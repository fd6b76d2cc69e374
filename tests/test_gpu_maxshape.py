"""GPU parity at the largest shapes the library accepts: d = f = 16384.

At this size every arithmetic path runs kernel variants that the production
shapes do not reach: the general fixed-point gate/up and down kernels with two
64-chunk steps per wave (eight steps per row), the fp32 gate/up with eight
waves per tile, both bf16 MFMA products with K = 16384 (256 groups), the
one-token router holding a full sixteen-float4 row slice per lane, and the
RMSNorm folded into that router.  Three experts (top-2) plus the shared one
keep the layer at 1.7 GB and the fp64 oracle at seconds per token.

The oracle runs once per module (route, weights, outputs, L1 norms of the
products) and every GPU call is checked against it: routing ids exactly (the
three tokens' k-th logit gaps are several units, far from the 1e-5 near-tie
rule), gate weights and logits within 1e-4 relative, union lists exactly,
outputs within |gpu - oracle| <= 1e-3 (1 + |oracle|) on the fp32 and
fixed-point paths and within 2e-2 of the L1 norm of the products on the bf16
path; one-token calls are bit-identical to the batched call.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAXW = synth.Workload(name="max16k", d=16384, f=16384, E=3, k=2, T=3, n_shared=1, seed=synth.BASE_SEED + 107)
AUTO, FP32, MFMA, FXP = 0, 1, 2, 3
EPS = 1e-6


@pytest.fixture(scope="module")
def maxrun():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    oracle.build(force=False)
    synth.build(force=False)
    w = MAXW
    need = (w.E + w.n_shared) * w.expert_bytes
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * need:
        pytest.skip("maximum-shape layer needs %.1f GB of device memory" % (need / 1e9))
    print("context", w.name, w.d, w.f, w.E, w.k, w.T, flush=True)
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=w.T)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    L, oidx, ow = ora.route(X)
    for t in range(w.T):
        s = np.sort(L[t])[::-1]
        assert s[w.k - 1] - s[w.k] > 1e-3, "token %d sits near a routing tie" % t
    out, l1 = ora.forward(X, oidx, ow)
    print("oracle done: max |out| %.4g, max L1 %.4g" % (np.abs(out).max(), l1.max()), flush=True)
    yield dict(ctx=ctx, ora=ora, X=X, L=L, idx=oidx, w=ow, out=out, l1=l1)
    ctx.close()
    del ctx
    torch.cuda.empty_cache()


def run_gpu(ctx, X, flags, one_call=False):
    xt = torch.from_numpy(np.ascontiguousarray(X, np.float32)).cuda()
    U = ctx.new_union(X.shape[0])
    res = xt.clone()
    logits = None
    if one_call:
        idx, wts = ctx.route_forward(0, xt, U, res, flags)
    else:
        idx, wts, logits = ctx.route(0, xt, U, want_logits=True)
        ctx.forward(0, xt, idx, wts, U, res, flags)
    ctx.sync()
    return dict(idx=idx.cpu().numpy(), w=wts.cpu().numpy(), out=res.cpu().numpy(), union=U.to_host(),
                logits=None if logits is None else logits.cpu().numpy())


def check_against_oracle(r, m, rows, what):
    assert np.array_equal(r["idx"], m["idx"][rows]), what + ": routing"
    P.assert_close(r["w"], m["w"][rows], rel=1e-4, what=what + ": gate weights")
    if r["logits"] is not None:
        P.assert_close(r["logits"], m["L"][rows], rel=1e-4, what=what + ": logits")
    ou = oracle.union(m["idx"][rows], MAXW.E)
    assert r["union"]["n_unique"] == ou["n_unique"], what + ": unique count"
    for key in ("ids", "offsets", "pair_token", "pair_slot", "pair_of"):
        assert np.array_equal(r["union"][key], ou[key]), what + ": union list " + key


def test_max_shape_fixed_point(maxrun):
    """AUTO picks the fixed-point path here; the batch and each token alone
    (route + forward, and the one-call form) match the oracle, and the
    one-token results equal the batched rows bit for bit."""
    m = maxrun
    batch = run_gpu(m["ctx"], m["X"], AUTO)
    check_against_oracle(batch, m, slice(None), "fxp batch")
    ratio = P.assert_close(batch["out"], m["out"], what="fxp batch output")
    forced = run_gpu(m["ctx"], m["X"], FXP)
    assert np.array_equal(forced["out"].view(np.uint32), batch["out"].view(np.uint32)), "AUTO is not the fxp path"
    for t in range(MAXW.T):
        rows = slice(t, t + 1)
        for one_call in (False, True):
            r = run_gpu(m["ctx"], m["X"][rows], FXP, one_call)
            check_against_oracle(r, m, rows, "fxp token %d" % t)
            assert np.array_equal(r["out"][0].view(np.uint32), batch["out"][t].view(np.uint32)), (t, one_call)
    print("max16k fixed point: worst |gpu-oracle|/bound %.3g" % ratio)


def test_max_shape_fp32(maxrun):
    m = maxrun
    r = run_gpu(m["ctx"], m["X"], FP32)
    check_against_oracle(r, m, slice(None), "fp32")
    ratio = P.assert_close(r["out"], m["out"], what="fp32 output")
    print("max16k fp32: worst |gpu-oracle|/bound %.3g" % ratio)


def test_max_shape_bf16_mfma(maxrun):
    m = maxrun
    r = run_gpu(m["ctx"], m["X"], MFMA)
    check_against_oracle(r, m, slice(None), "mfma")
    gpu = r["out"].astype(np.float64)
    assert np.all(np.isfinite(gpu))
    ratio = np.abs(gpu - m["out"]) / (2e-2 * m["l1"])
    assert ratio.max() <= 1.0, "mfma: max |gpu-oracle|/(2e-2 N) = %.3g" % ratio.max()
    print("max16k bf16 MFMA: worst ratio %.3g" % ratio.max())


def test_max_shape_rmsnorm_in_router(maxrun):
    """One stack step at d = 16384: colimoe_rmsnorm_route_forward (RMSNorm
    formed inside the one-token router) gives the bits of colimoe_rmsnorm +
    colimoe_route_forward, and its x matches the oracle's RMSNorm."""
    m = maxrun
    ctx = m["ctx"]
    r0 = m["X"][1:2] * 3.0
    ra = torch.from_numpy(np.ascontiguousarray(r0, np.float32)).cuda()
    rb = ra.clone()
    xa = torch.empty_like(ra)
    xb = torch.empty_like(ra)
    Ua, Ub = ctx.new_union(1), ctx.new_union(1)
    ctx.rmsnorm(ra, EPS, xa)
    ia, wa = ctx.route_forward(0, xa, Ua, ra, FXP)
    ib, wb = ctx.rmsnorm_route_forward(0, rb, EPS, xb, Ub, FXP)
    ctx.sync()
    assert np.array_equal(xa.cpu().numpy().view(np.uint32), xb.cpu().numpy().view(np.uint32))
    assert np.array_equal(ia.cpu().numpy(), ib.cpu().numpy())
    assert np.array_equal(wa.cpu().numpy().view(np.uint32), wb.cpu().numpy().view(np.uint32))
    assert np.array_equal(ra.cpu().numpy().view(np.uint32), rb.cpu().numpy().view(np.uint32))
    xo = oracle.rmsnorm(r0[0].astype(np.float64), EPS)
    P.assert_close(xb.cpu().numpy()[0], xo, what="RMSNorm at d = 16384")


# The expert-count limit (1024 experts, top-16, Zipf bias): sixteen keys per
# lane in the top-k, for one token (router + top-k + union in two launches),
# up to 16 tokens (top-k and union in one launch) and beyond (matrix-core
# router, separate top-k and union kernels).
MAXE = synth.Workload(name="e1024", d=256, f=128, E=1024, k=16, T=40, n_shared=1, zipf=1.1, rho=0.3,
                      seed=synth.BASE_SEED + 108)


def test_max_experts_top16():
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    oracle.build(force=False)
    synth.build(force=False)
    w = MAXE
    print("context", w.name, w.d, w.f, w.E, w.k, w.T, flush=True)
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=w.T)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    worst = 0.0
    for T in (w.T, 16, 5, 1):
        r = P.layer_parity(ctx, w, 0, X[:T], ora)
        worst = max(worst, r["ratio"])
        if T == 1:
            r1 = P.layer_parity(ctx, w, 0, X[:1], ora, one_call=True)
            assert np.array_equal(r1["out"].view(np.uint32), r["out"].view(np.uint32))
        print("e1024 T=%d: %d unique experts, near-tie tokens %s" % (T, r["union"]["n_unique"], r["differ"]))
    ctx.close()
    print("e1024: worst |gpu-oracle|/bound %.3g" % worst)

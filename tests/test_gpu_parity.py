"""GPU parity of the HIP path against the CPU oracle (fp32 path).

Bound per output: |gpu - oracle| <= 1e-3 * (1 + |oracle|).  Routing ids equal
the oracle's except on near-ties (gap < 1e-5 between the k-th and (k+1)-th
fp64 logits); union lists are compared exactly; batched results must be
bit-identical to one-at-a-time results.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
DECODE = synth.WORKLOADS["decode"]
UNION16 = synth.WORKLOADS["union16"]
# odd shapes: partial lane groups (d/32 = 10, f/32 = 6), E not a multiple of 64
RAGGED = synth.Workload(name="ragged", d=320, f=192, E=37, k=3, T=5, n_shared=1, zipf=1.1, rho=0.3,
                        seed=synth.BASE_SEED + 101)
# d/32 = 66: two chunk steps per row, the second one partial
RAGGED2 = synth.Workload(name="ragged2", d=2112, f=128, E=20, k=4, T=3, n_shared=0, seed=synth.BASE_SEED + 102)
# narrow rows of 33-63 chunks (d/32 = 46, f/32 = 34: 64 lanes per row in the
# narrow kernels), more experts than the one-launch small path takes
RAGGED4 = synth.Workload(name="ragged4", d=1472, f=1088, E=80, k=4, T=4, n_shared=1, zipf=1.1,
                         seed=synth.BASE_SEED + 104)
# wide in both d and f (fixed-point path) with partial steps in both GEMVs
RAGGED3 = synth.Workload(name="ragged3", d=2112, f=2112, E=24, k=3, T=4, n_shared=1, zipf=1.1, rho=0.5,
                         seed=synth.BASE_SEED + 103)
# wide, no shared expert, odd k: the few-token kernels' pair grids and token
# blocks without the shared rows
RAGGED5 = synth.Workload(name="ragged5", d=2112, f=2112, E=30, k=5, T=3, n_shared=0, zipf=1.1, rho=0.5,
                         seed=synth.BASE_SEED + 107)
FP32, FXP = 1, 3


def _ctx(w, n_layers=1, max_tokens=None):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, w.T, flush=True)
    return MoeContext(w.d, w.f, w.E, w.k, n_layers=n_layers, n_shared=w.n_shared,
                      max_tokens=max_tokens or max(w.T, 1))


@pytest.fixture(scope="module", autouse=True)
def _builds():
    oracle.build(force=False)
    synth.build(force=False)


def test_native_library_is_the_path():
    import int4_routed_expert_fp32_amd as cm
    L = cm.lib()
    assert L._name.endswith("libcolimoe.so")
    assert torch.cuda.is_available()


@pytest.mark.parametrize("w", [TINY, RAGGED, RAGGED2, DECODE], ids=lambda w: w.name)
def test_debug_expert_onehot_is_exact(w):
    """x = e_c makes g and u single dequantised weights q*s, exact in fp32."""
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    blob = synth.expert_blobs(w, 0, 3, 4)[0]
    Wg = oracle.dequant(*oracle.blob_sections(blob, w.d, w.f)[0], w.f, w.d)
    Wu = oracle.dequant(*oracle.blob_sections(blob, w.d, w.f)[1], w.f, w.d)
    for c in (0, 1, 33, w.d - 1):
        x = torch.zeros(w.d, dtype=torch.float32, device="cuda")
        x[c] = 1.0
        g, u, h, y = ctx.debug_expert(0, 3, x)
        assert np.array_equal(g.cpu().numpy().astype(np.float64), Wg[:, c])
        assert np.array_equal(u.cpu().numpy().astype(np.float64), Wu[:, c])


@pytest.mark.parametrize("w", [TINY, RAGGED, RAGGED2, DECODE], ids=lambda w: w.name)
def test_debug_expert_stages(w):
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    x = synth.activations(w, stream=7, T=1)[0]
    xt = torch.from_numpy(x).cuda()
    for e in ([0, w.E - 1] + ([-1] if w.n_shared else [])):
        blob = synth.expert_blobs(w, 0, e if e >= 0 else w.E, (e if e >= 0 else w.E) + 1)[0]
        o = oracle.expert(blob, w.d, w.f, x.astype(np.float64))
        g, u, h, y = (t.cpu().numpy() for t in ctx.debug_expert(0, e, xt))
        P.assert_close(g, o["g"], what="g")
        P.assert_close(u, o["u"], what="u")
        P.assert_close(h, o["h"], what="h")
        P.assert_close(y, o["y"], what="y")


def _rand_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (16, 256, 8), (7, 37, 3), (2048, 256, 8), (100, 16, 16),
                                   (64, 1000, 1), (65, 64, 2)])
def test_union_lists_exact(T, E, k):
    w = synth.Workload(name="u", d=256, f=128, E=E, k=k, T=T, n_shared=0)
    ctx = _ctx(w)
    rng = np.random.default_rng(T * 1000 + E + k)
    for trial in range(4):
        idx = _rand_routing(rng, T, E, k)
        if trial == 1:
            idx[:] = idx[0]  # identical tokens: U = k
        if trial == 3:
            idx[rng.random(idx.shape) < 0.3] = -1  # slots dropped by expert top-p: no pair
        U = ctx.new_union(T)
        ctx.union_build(torch.from_numpy(idx).cuda(), U)
        ctx.sync()
        g = U.to_host()
        o = oracle.union(idx, E)
        assert g["n_unique"] == o["n_unique"]
        for key in ("ids", "offsets", "pair_of"):
            assert np.array_equal(g[key], o[key]), key
        n = int(o["offsets"][-1])  # pairs listed (dropped slots have none)
        for key in ("pair_token", "pair_slot"):
            assert np.array_equal(g[key][:n], o[key][:n]), key


def test_invalid_routing_is_reported():
    """An id outside [0, E) other than -1, or an expert twice in one token, is
    an invalid routing: empty lists and E_ARG at the next sync.  -1 is a
    dropped slot (expert top-p), not an error, also twice in one token."""
    w = TINY
    ctx = _ctx(w, max_tokens=2)
    U = ctx.new_union(2)
    for bad in (np.array([[0, 16], [1, 2]], np.int32), np.array([[3, 3], [1, 2]], np.int32),
                np.array([[-2, 2], [1, 2]], np.int32)):
        ctx.union_build(torch.from_numpy(bad).cuda(), U)
        assert ctx.sync(check=False) == -1
        assert int(U.n_unique.item()) == 0
    assert ctx.sync(check=False) == 0
    for ok in (np.array([[-1, 2], [1, 2]], np.int32), np.array([[-1, -1], [5, -1]], np.int32)):
        ctx.union_build(torch.from_numpy(ok).cuda(), U)
        assert ctx.sync(check=False) == 0
        g, o = U.to_host(), oracle.union(ok, w.E)
        assert g["n_unique"] == o["n_unique"]
        for key in ("ids", "offsets", "pair_of"):
            assert np.array_equal(g[key], o[key]), key


@pytest.mark.parametrize("w", [TINY, RAGGED, RAGGED2, RAGGED3, RAGGED4, RAGGED5], ids=lambda w: w.name)
def test_layer_parity_small(w):
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    r = P.layer_parity(ctx, w, 0, X, ora)
    if w is RAGGED3:  # both arithmetic paths, and the one-call entry point
        r2 = P.layer_parity(ctx, w, 0, X, ora, flags=FP32)
        r3 = P.layer_parity(ctx, w, 0, X, ora, one_call=True)
        assert np.array_equal(r3["out"].view(np.uint32), r["out"].view(np.uint32))
        print("ragged3 fp32 path worst ratio", r2["ratio"])
    if w is RAGGED4:  # every token alone (one call) gives its row of the batch
        for t in range(w.T):
            a = P.layer_parity(ctx, w, 0, X[t:t + 1], ora, one_call=True)
            assert np.array_equal(a["out"][0].view(np.uint32), r["out"][t].view(np.uint32)), t
    if w is RAGGED5:  # both paths, one call, and every token alone = its row of the batch
        for flags in (FXP, FP32):
            b = P.layer_parity(ctx, w, 0, X, ora, flags=flags, one_call=True)
            for t in range(w.T):
                a = P.layer_parity(ctx, w, 0, X[t:t + 1], ora, flags=flags, one_call=True)
                assert np.array_equal(a["out"][0].view(np.uint32), b["out"][t].view(np.uint32)), (flags, t)
            print("ragged5 flags", flags, "worst ratio", b["ratio"])
    print(w.name, "worst ratio", r["ratio"], "near-tie tokens", r["differ"])
    # union lists from route equal the oracle's union of the GPU routing
    o = oracle.union(r["idx"], w.E)
    for key in ("ids", "offsets"):
        assert np.array_equal(r["union"][key], o[key])


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
def test_layer_parity_decode(flags):
    w = DECODE
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    for stream in (0, 1, 2):
        X = synth.activations(w, stream=stream)
        r = P.layer_parity(ctx, w, 0, X, ora, flags=flags)
        r1 = P.layer_parity(ctx, w, 0, X, ora, flags=flags, one_call=True)
        assert np.array_equal(r1["out"].view(np.uint32), r["out"].view(np.uint32))
        print("decode", flags, "stream", stream, "worst ratio", r["ratio"], "near-ties", r["differ"])


def test_zero_tokens_is_a_noop():
    w = TINY
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    x = torch.zeros((0, w.d), dtype=torch.float32, device="cuda")
    idx, wts, _ = ctx.route(0, x)
    res = torch.zeros((0, w.d), dtype=torch.float32, device="cuda")
    ctx.forward(0, x, idx, wts, None, res)
    ctx.sync()


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
def test_union16_parity_and_batch_identity(flags):
    """16 correlated positions: batched == one at a time, bit for bit; each
    unique expert appears once in the union; outputs match the oracle."""
    w = UNION16
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=0)
    r = P.layer_parity(ctx, w, 0, X, ora, flags=flags)
    nu = r["union"]["n_unique"]
    print("union16: unique experts", nu, "of", w.T * w.k, "pairs; worst ratio", r["ratio"])
    assert nu < w.T * w.k
    xt = torch.from_numpy(X).cuda()
    for t in range(w.T):
        x1 = xt[t:t + 1].contiguous()
        U1 = ctx.new_union(1)
        idx1, w1, _ = ctx.route(0, x1, U1)
        res1 = x1.clone()
        ctx.forward(0, x1, idx1, w1, U1, res1, flags)
        ctx.sync()
        assert np.array_equal(idx1.cpu().numpy()[0], r["idx"][t])
        assert np.array_equal(w1.cpu().numpy()[0].view(np.uint32), r["w"][t].view(np.uint32))
        assert np.array_equal(res1.cpu().numpy()[0].view(np.uint32), r["out"][t].view(np.uint32)), t


@pytest.mark.parametrize("T", [2, 3, 4])
def test_verify_positions_match_single_token_calls(T):
    """A few draft positions in one call (the batch-union path) give each
    position the bits of a one-token call (the one-token kernels), through
    colimoe_route_forward both times, and match the oracle."""
    w = synth.WORKLOADS["verify4"].with_(T=T)
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=7)
    r = P.layer_parity(ctx, w, 0, X, ora, one_call=True)
    for t in range(T):
        a = P.layer_parity(ctx, w, 0, X[t:t + 1], ora, one_call=True)
        assert np.array_equal(a["idx"][0], r["idx"][t])
        assert np.array_equal(a["out"][0].view(np.uint32), r["out"][t].view(np.uint32)), t
    print("verify T=%d: unique experts %d, worst ratio %.3g" % (T, r["union"]["n_unique"], r["ratio"]))


def test_forced_routing_onehot_gate():
    """Caller-forced routing with gate weights (1, 0, ...) and a zero residual
    yields exactly one expert's output (plus the shared expert)."""
    w = RAGGED
    ctx = _ctx(w, max_tokens=1)
    P.load_layer(ctx, w, 0)
    x = synth.activations(w, stream=3, T=1)
    xt = torch.from_numpy(x).cuda()
    idx = torch.tensor([[5, 0, 9]], dtype=torch.int32, device="cuda")
    wts = torch.tensor([[1.0, 0.0, 0.0]], dtype=torch.float32, device="cuda")
    res = torch.zeros_like(xt)
    ctx.forward(0, xt, idx, wts, None, res)
    ctx.sync()
    ora = P.OracleLayer(w, 0)
    out, _ = ora.forward(x, np.array([[5, 0, 9]]), np.array([[1.0, 0.0, 0.0]]), residual=np.zeros_like(x))
    P.assert_close(res.cpu().numpy(), out, what="one-hot gate")


# One-token shapes that reach the other kernel variants: two steps per row with
# a partial second one (d = f = 2112: the streaming down kernel, and the lanes
# past the row end of the fp32 one-token pair), 17 slots (k = 16 + shared:
# more slots than one block of slot-waves holds), and d > 8192 (the general
# fixed-point and fp32 kernels).
DEC_SHAPES = [
    synth.Workload(name="dec_2step", d=2112, f=2112, E=40, k=3, T=3, n_shared=1, zipf=1.1,
                   seed=synth.BASE_SEED + 104),
    synth.Workload(name="dec_k16", d=2048, f=2048, E=64, k=16, T=3, n_shared=1, seed=synth.BASE_SEED + 105),
    synth.Workload(name="dec_wide", d=8256, f=2048, E=16, k=2, T=3, n_shared=1, seed=synth.BASE_SEED + 106),
]


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
@pytest.mark.parametrize("w", DEC_SHAPES, ids=lambda w: w.name)
def test_one_token_kernel_variants(w, flags):
    """Each token alone (one call and route + forward) matches the oracle, the
    two call forms agree bit for bit, and both equal the batched call."""
    ctx = _ctx(w)
    P.load_layer(ctx, w, 0)
    ora = P.OracleLayer(w, 0)
    X = synth.activations(w, stream=4)
    batch = P.layer_parity(ctx, w, 0, X, ora, flags=flags)
    for t in range(w.T):
        x1 = X[t:t + 1]
        a = P.layer_parity(ctx, w, 0, x1, ora, flags=flags, one_call=True)
        b = P.layer_parity(ctx, w, 0, x1, ora, flags=flags)
        assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32)), t
        assert np.array_equal(a["out"][0].view(np.uint32), batch["out"][t].view(np.uint32)), t
        assert np.array_equal(a["idx"][0], batch["idx"][t])
    print(w.name, "worst ratio", batch["ratio"])


@pytest.mark.parametrize("flags", [FXP, FP32, 2], ids=["fxp", "fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("bad", ["nan", "inf"])
def test_non_finite_inputs_propagate(flags, T, bad):
    """One NaN or one infinity in a token's activations makes every output of
    that token non-finite on every arithmetic path (the fixed-point encoding
    gives the affected group a NaN scale instead of a finite digit pattern;
    [A] §4: precision never changes silently).  The other tokens are
    untouched: their bits equal those of a call without the bad value."""
    w = RAGGED3
    ctx = _ctx(w, max_tokens=3)
    P.load_layer(ctx, w, 0)
    X = synth.activations(w, stream=11)[:T].copy()
    rng = np.random.default_rng(5)
    idx = torch.from_numpy(np.stack([rng.permutation(w.E)[:w.k] for _ in range(T)]).astype(np.int32)).cuda()
    wts = torch.full((T, w.k), 1.0 / w.k, dtype=torch.float32, device="cuda")

    def run(Xh):
        x = torch.from_numpy(np.ascontiguousarray(Xh)).cuda()
        res = x.clone()
        ctx.forward(0, x, idx, wts, None, res, flags)
        ctx.sync()
        return res.cpu().numpy()

    clean = run(X)
    assert np.all(np.isfinite(clean))
    Xb = X.copy()
    Xb[T - 1, 1000] = np.nan if bad == "nan" else np.inf
    out = run(Xb)
    # the residual keeps the token's own input; every other output is non-finite
    mask = np.ones(w.d, bool)
    mask[1000] = False
    assert not np.any(np.isfinite(out[T - 1][mask])), "finite outputs from a %s input" % bad
    if T > 1:
        assert np.array_equal(out[:T - 1].view(np.uint32), clean[:T - 1].view(np.uint32))

"""Tiered placement: layers whose routed experts stay in pinned host memory
and move into a small HBM expert cache on demand (least recently used out).
The same calls on the same layers loaded into HBM give the same bits; a call
that needs more experts than the cache holds is refused; the cache counts
its hits and misses.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FP32, FXP = 1, 3
W = synth.Workload(name="tiered", d=6144, f=2048, E=32, k=8, T=2, n_shared=1, zipf=1.1,
                   seed=synth.BASE_SEED + 301)
SLOTS = 12  # two pinned shared experts + 10: at most 10 routed experts per call


def _ctx(n_layers=2):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    return MoeContext(W.d, W.f, W.E, W.k, n_layers=n_layers, n_shared=W.n_shared, max_tokens=W.T)


@pytest.fixture(scope="module")
def pair():
    oracle.build(force=False)
    synth.build(force=False)
    dev, host = _ctx(), _ctx()
    host.set_expert_cache(SLOTS)
    for l in range(2):
        args = (synth.router(W, l), synth.bias(W, l), synth.expert_blobs(W, l, 0, W.E), synth.shared_blob(W, l))
        dev.load_layer(l, *args)
        host.load_layer_host(l, *args)
    print("tiered: 2 layers, %d experts each, cache of %d slots" % (W.E, SLOTS), flush=True)
    yield dev, host
    dev.close()
    host.close()


def _call(ctx, layer, x, flags):
    U = ctx.new_union(x.shape[0])
    res = x.clone()
    idx, w = ctx.route_forward(layer, x, U, res, flags)
    ctx.sync()
    return idx.cpu().numpy(), w.cpu().numpy().view(np.uint32), res.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
def test_host_layers_match_hbm_layers(pair, flags):
    dev, host = pair
    h0, m0, slots = host.cache_stats()
    assert slots == SLOTS
    X = torch.from_numpy(synth.activations(W.with_(T=16), stream=41)).cuda()
    for t in range(16):
        x = X[t:t + 1].contiguous()
        a = _call(dev, t % 2, x, flags)
        b = _call(host, t % 2, x, flags)
        for u, v in zip(a, b):
            assert np.array_equal(u, v), t
    h1, m1, _ = host.cache_stats()
    print("tiered %d: hits %d misses %d" % (flags, h1 - h0, m1 - m0))
    assert (h1 - h0) + (m1 - m0) == 16 * W.k
    assert m1 - m0 >= 10  # the cache is far smaller than the two layers' 64 experts


def test_host_layer_stack_step_and_batch(pair):
    dev, host = pair
    R = torch.from_numpy(synth.activations(W.with_(T=2), stream=42) * 2.0).cuda()
    for layer in (0, 1):
        r1, r2 = R[:1].clone(), R[:1].clone()
        x1, x2 = torch.empty_like(r1), torch.empty_like(r2)
        i1, w1 = dev.rmsnorm_route_forward(layer, r1, 1e-6, x1, dev.new_union(1), FXP)
        i2, w2 = host.rmsnorm_route_forward(layer, r2, 1e-6, x2, host.new_union(1), FXP)
        dev.sync()
        host.sync()
        assert torch.equal(i1, i2) and torch.equal(r1, r2) and torch.equal(x1, x2)
    # two tokens in one call: served if their union fits the free slots, refused otherwise
    import int4_routed_expert_fp32_amd as cm
    x = R.contiguous()
    U = dev.new_union(2)
    idx, _, _ = dev.route(0, x, U)
    dev.sync()
    nu = int(U.n_unique.item())
    a = _call(dev, 0, x, FXP)
    U2 = host.new_union(2)
    idx2 = torch.empty((2, W.k), dtype=torch.int32, device="cuda")
    w2 = torch.empty((2, W.k), dtype=torch.float32, device="cuda")
    res = x.clone()
    rc = cm.colimoe_route_forward(host.ctx, 0, x.data_ptr(), 2, idx2.data_ptr(), w2.data_ptr(), U2.abi(),
                                  res.data_ptr(), FXP, check=False)
    host.sync()
    print("two tokens: %d distinct experts, rc %d" % (nu, rc))
    if nu <= SLOTS - 2:
        assert rc == 0 and np.array_equal(res.cpu().numpy().view(np.uint32), a[2])
    else:
        assert rc == cm.COLIMOE_E_WORKSPACE


def test_host_layer_matches_oracle(pair):
    dev, host = pair
    ora = P.OracleLayer(W, 1)
    X = synth.activations(W.with_(T=1), stream=43)
    r = P.layer_parity(host, W, 1, X, ora, flags=FXP, one_call=True)
    print("tiered vs oracle: worst ratio", r["ratio"])


def test_debug_expert_refused_on_host_layer(pair):
    import int4_routed_expert_fp32_amd as cm
    dev, host = pair
    x = torch.zeros(W.d, dtype=torch.float32, device="cuda")
    g = torch.empty(W.f, dtype=torch.float32, device="cuda")
    y = torch.empty(W.d, dtype=torch.float32, device="cuda")
    rc = cm.lib().colimoe_debug_expert(host.ctx, 0, 3, x.data_ptr(), g.data_ptr(), g.data_ptr(), g.data_ptr(),
                                       y.data_ptr())
    assert rc == cm.COLIMOE_E_STATE


def test_repin_keeps_results_and_pins(pair):
    import int4_routed_expert_fp32_amd as cm
    dev, host = pair
    assert cm.colimoe_cache_repin(host.ctx, SLOTS, check=False) == cm.COLIMOE_E_WORKSPACE
    host.cache_repin(2)  # the two experts the earlier calls needed most stay put
    X = torch.from_numpy(synth.activations(W.with_(T=8), stream=44)).cuda()
    h0, m0, _ = host.cache_stats()
    for t in range(8):
        x = X[t:t + 1].contiguous()
        a = _call(dev, t % 2, x, FXP)
        b = _call(host, t % 2, x, FXP)
        for u, v in zip(a, b):
            assert np.array_equal(u, v), t
    h1, m1, _ = host.cache_stats()
    print("after repin: hits %d misses %d" % (h1 - h0, m1 - m0))
    host.cache_repin(0)

"""Tiered placement: layers whose routed experts stay in pinned host memory and
move into an HBM expert cache on demand, split into per-layer partitions
with their own least-recently-used order ([A] §2), learned pinning from a
usage histogram that can be saved and loaded, automatic repinning every N
tokens ([D] key tuning parameters, --repin N), and the next layer's router run
one layer ahead to prefetch its predicted experts ([A] §2).

The cache never changes results: the same calls on the same layers loaded
into HBM give the same bits, with and without prefetch, pinning or automatic
repinning.  A call that needs more evictable slots than its layer's partition
has is refused.
"""
import os
import tempfile

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
SLOTS = 24  # two layers: 12 slots each, the shared expert and 11 routed experts
PER_LAYER = 12
MAX_PIN = PER_LAYER - 1 - W.k


def _ctx(n_layers=2):
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    return MoeContext(W.d, W.f, W.E, W.k, n_layers=n_layers, n_shared=W.n_shared, max_tokens=W.T)


def _layer_args(l):
    return (synth.router(W, l), synth.bias(W, l), synth.expert_blobs(W, l, 0, W.E), synth.shared_blob(W, l))


@pytest.fixture(scope="module")
def pair():
    oracle.build(force=False)
    synth.build(force=False)
    dev = _ctx()
    for l in range(2):
        dev.load_layer(l, *_layer_args(l))
    print("tiered: 2 layers, %d experts each, cache of %d slots" % (W.E, SLOTS), flush=True)
    yield dev
    dev.close()


def _host_ctx():
    host = _ctx()
    host.set_expert_cache(SLOTS)
    for l in range(2):
        host.load_layer_host(l, *_layer_args(l))
    return host


@pytest.fixture()
def host():
    h = _host_ctx()
    yield h
    h.close()


def _call(ctx, layer, x, flags):
    U = ctx.new_union(x.shape[0])
    res = x.clone()
    idx, w = ctx.route_forward(layer, x, U, res, flags)
    ctx.sync()
    return idx.cpu().numpy(), w.cpu().numpy().view(np.uint32), res.cpu().numpy().view(np.uint32)


def _same(a, b, what):
    for u, v in zip(a, b):
        assert np.array_equal(u, v), what


@pytest.mark.parametrize("prefetch", [0, 3, W.k], ids=["lru", "prefetch3", "prefetch8"])
@pytest.mark.parametrize("flags", [FXP, FP32], ids=["fxp", "fp32"])
def test_host_layers_match_hbm_layers(pair, host, flags, prefetch):
    dev = pair
    host.cache_set_prefetch(prefetch)
    import int4_routed_expert_fp32_amd as cm
    assert cm.colimoe_cache_set_prefetch(host.ctx, W.k + 1, check=False) == cm.COLIMOE_E_ARG
    info = host.cache_info()
    assert info.slots == SLOTS and info.slots_per_layer == PER_LAYER
    X = torch.from_numpy(synth.activations(W.with_(T=16), stream=41)).cuda()
    for t in range(16):
        x = X[t:t + 1].contiguous()
        _same(_call(dev, t % 2, x, flags), _call(host, t % 2, x, flags), "token %d" % t)
    info = host.cache_info()
    print("tiered %d prefetch %s: hits %d misses %d predicted %d (hits %d) prefetched %d (used %d)" % (
        flags, prefetch, info.hits, info.misses, info.predicted, info.predicted_hits, info.prefetched,
        info.prefetched_used))
    assert info.hits + info.misses == 16 * W.k
    assert info.misses >= 10  # each partition holds 11 of its layer's 32 routed experts
    if prefetch:
        # every layer-1 call followed a layer-0 call that predicted it
        assert info.predicted == 8 * W.k
        assert 0 <= info.predicted_hits <= info.predicted
        assert 0 <= info.prefetched_used <= info.prefetched <= 8 * prefetch
    else:
        assert info.predicted == 0 and info.prefetched == 0


def test_partitions_are_per_layer(host):
    """A layer's calls evict only its own experts: layer 1's experts survive
    many layer-0 calls."""
    X = torch.from_numpy(synth.activations(W.with_(T=12), stream=45)).cuda()
    x1 = X[0:1].contiguous()
    _call(host, 1, x1, FXP)
    for t in range(1, 12):
        _call(host, 0, X[t:t + 1].contiguous(), FXP)
    before = host.cache_info()
    _call(host, 1, x1, FXP)
    after = host.cache_info()
    assert after.misses == before.misses and after.hits == before.hits + W.k


def test_host_layer_stack_step_and_batch(pair, host):
    dev = pair
    R = torch.from_numpy(synth.activations(W.with_(T=2), stream=42) * 2.0).cuda()
    for layer in (0, 1):
        r1, r2 = R[:1].clone(), R[:1].clone()
        x1, x2 = torch.empty_like(r1), torch.empty_like(r2)
        i1, w1 = dev.rmsnorm_route_forward(layer, r1, 1e-6, x1, dev.new_union(1), FXP)
        i2, w2 = host.rmsnorm_route_forward(layer, r2, 1e-6, x2, host.new_union(1), FXP)
        dev.sync()
        host.sync()
        assert torch.equal(i1, i2) and torch.equal(r1, r2) and torch.equal(x1, x2)
    # two tokens in one call: served if their union fits the partition's evictable slots, refused otherwise
    import int4_routed_expert_fp32_amd as cm
    x = R.contiguous()
    U = dev.new_union(2)
    dev.route(0, x, U)
    dev.sync()
    nu = int(U.n_unique.item())
    a = _call(dev, 0, x, FXP)
    idx2 = torch.empty((2, W.k), dtype=torch.int32, device="cuda")
    w2 = torch.empty((2, W.k), dtype=torch.float32, device="cuda")
    res = x.clone()
    rc = cm.colimoe_route_forward(host.ctx, 0, x.data_ptr(), 2, idx2.data_ptr(), w2.data_ptr(), host.new_union(2).abi(),
                                  res.data_ptr(), FXP, check=False)
    host.sync()
    print("two tokens: %d distinct experts, rc %d" % (nu, rc))
    if nu <= PER_LAYER - 1:
        assert rc == 0 and np.array_equal(res.cpu().numpy().view(np.uint32), a[2])
    else:
        assert rc == cm.COLIMOE_E_WORKSPACE


def test_host_layer_matches_oracle(host):
    ora = P.OracleLayer(W, 1)
    X = synth.activations(W.with_(T=1), stream=43)
    r = P.layer_parity(host, W, 1, X, ora, flags=FXP, one_call=True)
    print("tiered vs oracle: worst ratio", r["ratio"])


def test_debug_expert_refused_on_host_layer(host):
    import int4_routed_expert_fp32_amd as cm
    x = torch.zeros(W.d, dtype=torch.float32, device="cuda")
    g = torch.empty(W.f, dtype=torch.float32, device="cuda")
    y = torch.empty(W.d, dtype=torch.float32, device="cuda")
    rc = cm.lib().colimoe_debug_expert(host.ctx, 0, 3, x.data_ptr(), g.data_ptr(), g.data_ptr(), g.data_ptr(),
                                       y.data_ptr())
    assert rc == cm.COLIMOE_E_STATE


def test_repin_to_the_limit_then_two_tokens(pair, host):
    """After pinning the most experts the partitions allow, a call whose
    misses fit the remaining evictable slots still runs (pinned hits do not
    count against them) and gives the HBM-resident bits."""
    import int4_routed_expert_fp32_amd as cm
    dev = pair
    assert cm.colimoe_cache_repin(host.ctx, MAX_PIN + 1, check=False) == cm.COLIMOE_E_WORKSPACE
    X = torch.from_numpy(synth.activations(W.with_(T=8), stream=44)).cuda()
    for t in range(8):
        _call(host, t % 2, X[t:t + 1].contiguous(), FXP)
    host.cache_repin(MAX_PIN)
    assert host.cache_info().pinned == 2 * MAX_PIN
    # two copies of one token: 8 distinct experts, at most 8 of them outside the pins
    x2 = torch.cat([X[0:1], X[0:1]]).contiguous()
    _same(_call(dev, 0, x2, FXP), _call(host, 0, x2, FXP), "two tokens after repin")
    for t in range(8):
        x = X[t:t + 1].contiguous()
        _same(_call(dev, t % 2, x, FXP), _call(host, t % 2, x, FXP), "token %d after repin" % t)
    host.cache_repin(0)
    assert host.cache_info().pinned == 0


def test_usage_histogram_save_and_load(host):
    """The usage histogram counts the tokens routed to each expert; saved to a
    file and loaded into a fresh context it gives the same counts and the same
    pins."""
    import int4_routed_expert_fp32_amd as cm
    X = torch.from_numpy(synth.activations(W.with_(T=10), stream=46)).cuda()
    counts = np.zeros((2, W.E), np.uint32)
    for t in range(10):
        idx, _, _ = _call(host, t % 2, X[t:t + 1].contiguous(), FXP)
        np.add.at(counts[t % 2], idx.ravel(), 1)
    for l in range(2):
        assert np.array_equal(host.cache_usage(l), counts[l])
    host.cache_repin(MAX_PIN)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "usage.bin")
        host.cache_usage_save(path)
        assert os.path.getsize(path) == 16 + 4 * 2 * W.E
        other = _host_ctx()
        try:
            other.cache_usage_load(path)
            for l in range(2):
                assert np.array_equal(other.cache_usage(l), counts[l])
            other.cache_repin(MAX_PIN)
            assert other.cache_info().pinned == host.cache_info().pinned
            # a file of another shape, and a file that is not a usage file
            bad = os.path.join(d, "bad.bin")
            with open(path, "rb") as f:
                raw = bytearray(f.read())
            raw[12:16] = np.int32(W.E + 1).tobytes()
            with open(bad, "wb") as f:
                f.write(raw)
            assert cm.colimoe_cache_usage_load(other.ctx, bad, check=False) == cm.COLIMOE_E_SHAPE
            with open(bad, "wb") as f:
                f.write(b"not a usage histogram")
            assert cm.colimoe_cache_usage_load(other.ctx, bad, check=False) == cm.COLIMOE_E_ARG
            assert np.array_equal(other.cache_usage(0), counts[0])  # a refused load changes nothing
        finally:
            other.close()


def test_autorepin(pair, host):
    """Every 4 tokens of a layer, its next call repins it by itself; results
    stay those of the HBM-resident layers."""
    import int4_routed_expert_fp32_amd as cm
    dev = pair
    assert cm.colimoe_cache_set_autorepin(host.ctx, 4, MAX_PIN + 1, check=False) == cm.COLIMOE_E_WORKSPACE
    host.cache_set_autorepin(4, MAX_PIN)
    X = torch.from_numpy(synth.activations(W.with_(T=12), stream=47)).cuda()
    pinned = []
    for t in range(12):
        x = X[t:t + 1].contiguous()
        _same(_call(dev, t % 2, x, FXP), _call(host, t % 2, x, FXP), "token %d" % t)
        pinned.append(host.cache_info().pinned)
    print("pinned slots after each token:", pinned)
    # layer 0 repins at its 4th token (t = 6), layer 1 at its 4th (t = 7)
    assert pinned[5] == 0 and pinned[6] == MAX_PIN and pinned[7] == 2 * MAX_PIN


def test_prefetch_through_the_stack_step(pair, host):
    """The stacked-layer call on host-resident layers with prefetch: layer 0's
    call predicts layer 1 from its input; bits equal the HBM-resident ones."""
    dev = pair
    host.cache_set_prefetch(W.k)
    R = torch.from_numpy(synth.activations(W.with_(T=8), stream=48)).cuda()
    for t in range(8):
        rd, rh = R[t:t + 1].clone(), R[t:t + 1].clone()
        xd, xh = torch.empty_like(rd), torch.empty_like(rh)
        for layer in (0, 1):
            i1, _ = dev.rmsnorm_route_forward(layer, rd, 1e-6, xd, dev.new_union(1), FXP)
            i2, _ = host.rmsnorm_route_forward(layer, rh, 1e-6, xh, host.new_union(1), FXP)
        dev.sync()
        host.sync()
        assert torch.equal(rd, rh) and torch.equal(xd, xh) and torch.equal(i1, i2)
    info = host.cache_info()
    print("stack prefetch: predicted %d, named %d (%.2f), prefetched %d, used %d" % (
        info.predicted, info.predicted_hits, info.predicted_hits / max(info.predicted, 1), info.prefetched,
        info.prefetched_used))
    assert info.predicted == 8 * W.k

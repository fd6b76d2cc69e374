"""Pins of the CPU oracle against things other than itself.

Each check below compares the oracle with a value fixed by a definition, a
library routine, a closed form, an invariant, brute force, an exact sum or a
size the colibrì pages print.  ``test_planted_mistakes_are_caught`` builds
copies of the oracle with one plausible mistake planted in each
(``tests/_mutants.py``, on the CPU) and requires each copy to fail at least
one pin.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from tests import _dense, _mutants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)
    synth.build(force=False)
    yield


def _tiny_inputs(layer=0):
    blobs = synth.expert_blobs(TINY, layer, 0, TINY.E)
    R = synth.router(TINY, layer)
    x = synth.activations(TINY, stream=layer)
    return blobs, R, x


def _rand_blob(rng, d, f):
    nb = oracle.expert_bytes(d, f)
    blob = rng.integers(0, 256, nb, dtype=np.uint8)
    # overwrite the scale sections with valid positive fp16 values
    for (n, s) in _dense.sections(blob, d, f):
        pass
    w = d * f
    o = 0
    for _ in range(3):
        o += w // 2
        ns = w // 64
        sc = rng.uniform(0.005, 0.02, ns).astype(np.float16).view(np.uint8)
        blob[o:o + 2 * ns] = sc
        o += 2 * ns
    return blob


# ---------------------------------------------------------------- decoding

def pin_nibble_table():
    for b in range(256):
        lo = int(np.int8(np.uint8((b << 4) & 0xFF)) >> 4)
        hi = int(np.int8(np.uint8(b)) >> 4)
        assert oracle.nibble(b, False) == lo, b
        assert oracle.nibble(b, True) == hi, b
    # hand-packed bytes: (even element, odd element)
    for b, (e0, e1) in {0x8F: (-1, -8), 0x70: (0, 7), 0x08: (-8, 0), 0xFF: (-1, -1), 0x00: (0, 0),
                        0x17: (7, 1)}.items():
        assert (oracle.nibble(b, False), oracle.nibble(b, True)) == (e0, e1), hex(b)


def test_nibble_table():
    pin_nibble_table()


def pin_half_table():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert oracle.half(0x3C00) == 1.0
    assert oracle.half(0x1E66) == 0.0062484741210937500
    assert oracle.half(0x0001) == 2.0 ** -24


def test_half_table():
    pin_half_table()


def pin_dequant_matches_numpy():
    rng = np.random.default_rng(1)
    rows, cols = 8, 256
    nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, rows * cols // 64).astype(np.float16).view(np.uint8)
    W = oracle.dequant(nib, sc, rows, cols)
    assert np.array_equal(W, _dense.dense_matrix(nib, sc, rows, cols))


def test_dequant_matches_numpy():
    pin_dequant_matches_numpy()


def _const_row(v, rows, cols, s_bits):
    nibv = v & 15
    nib = np.full(rows * cols // 2, nibv | (nibv << 4), dtype=np.uint8)
    sc = np.full(rows * cols // 64, s_bits, dtype=np.uint16).view(np.uint8)
    return nib, sc


def pin_matvec_closed_forms():
    rows, cols = 4, 192
    x = np.random.default_rng(2).standard_normal(cols).astype(np.float32).astype(np.float64)
    for v in (-8, -3, 0, 5, 7):
        for s_bits in (0x3C00, 0x1E66, 0x2400):
            s = float(np.uint16(s_bits).view(np.float16))
            nib, sc = _const_row(v, rows, cols, s_bits)
            y, _ = oracle.matvec(nib, sc, rows, cols, x)
            exact = Fraction(v) * Fraction(s) * sum(Fraction(float(t)) for t in x)
            for r in range(rows):
                assert abs(Fraction(y[r]) - exact) <= Fraction(cols * 2.0 ** -52) * abs(v * s) * np.abs(x).sum() + \
                    Fraction(2.0 ** -1074)
    # one-hot input picks a column: exact q * s
    rng = np.random.default_rng(3)
    nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, rows * cols // 64).astype(np.float16).view(np.uint8)
    Wn = _dense.dense_matrix(nib, sc, rows, cols)
    for c in (0, 1, 63, 64, 127, 191):
        e = np.zeros(cols)
        e[c] = 1.0
        y, _ = oracle.matvec(nib, sc, rows, cols, e)
        assert np.array_equal(y, Wn[:, c])
    # doubling every scale (exponent + 1) doubles the output exactly
    x2 = rng.standard_normal(cols).astype(np.float32).astype(np.float64)
    y1, _ = oracle.matvec(nib, sc, rows, cols, x2)
    sc2 = (sc.view(np.uint16) + np.uint16(0x0400)).view(np.uint8)
    y2, _ = oracle.matvec(nib, sc2, rows, cols, x2)
    assert np.array_equal(y2, 2.0 * y1)


def test_matvec_closed_forms():
    pin_matvec_closed_forms()


def pin_matvec_exact_sum():
    """fp32 inputs times int4*fp16 weights are exact in fp64; the oracle's
    sequential sum must lie within n*u*sum|p| of the exact sum."""
    rng = np.random.default_rng(4)
    rows, cols = 6, 512
    nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, rows * cols // 64).astype(np.float16).view(np.uint8)
    x = rng.standard_normal(cols).astype(np.float32).astype(np.float64)
    y, yabs = oracle.matvec(nib, sc, rows, cols, x)
    W = _dense.dense_matrix(nib, sc, rows, cols)
    for r in range(rows):
        prods = [Fraction(float(W[r, c])) * Fraction(float(x[c])) for c in range(cols)]
        exact = sum(prods)
        sabs = sum(abs(p) for p in prods)
        assert abs(Fraction(y[r]) - exact) <= Fraction(cols) * Fraction(2.0 ** -53) * sabs
        assert abs(Fraction(yabs[r]) - sabs) <= Fraction(cols) * Fraction(2.0 ** -53) * sabs


def test_matvec_exact_sum():
    pin_matvec_exact_sum()


# ------------------------------------------------------------------ router

def pin_router():
    blobs, R, x = _tiny_inputs()
    bias = synth.bias(synth.WORKLOADS["union16"].with_(E=TINY.E, d=TINY.d), 0)
    for c in (0, 5, 255):
        e = np.zeros(TINY.d)
        e[c] = 1.0
        l = oracle.router(R, bias, e)
        assert np.array_equal(l, R[:, c].astype(np.float64) + bias.astype(np.float64))
    l = oracle.router(R, None, x[0].astype(np.float64))
    for ei in range(TINY.E):
        ex = math.fsum(float(R[ei, c]) * float(x[0, c]) for c in range(TINY.d))
        assert abs(l[ei] - ex) <= TINY.d * 2.0 ** -53 * np.abs(R[ei].astype(np.float64) * x[0]).sum()


def test_router():
    pin_router()


def _lib_topk(l, k):
    return np.lexsort((np.arange(l.size), -l))[:k].astype(np.int32)


def pin_topk():
    rng = np.random.default_rng(5)
    for trial in range(200):
        E = int(rng.integers(2, 300))
        k = int(rng.integers(1, min(E, 16) + 1))
        l = rng.standard_normal(E)
        if trial % 3 == 0:  # inject exact ties
            l = np.round(l * 2) / 2
        ref = _lib_topk(l, k)
        assert np.array_equal(oracle.topk_sort(l, k), ref)
        assert np.array_equal(oracle.topk_select(l, k), ref)
    # all equal: lowest indices, uniform weights
    l = np.full(256, 0.25)
    idx = oracle.topk_sort(l, 8)
    assert list(idx) == list(range(8))
    w = oracle.softmax_selected(l, idx)
    assert np.allclose(w, 1 / 8, rtol=0, atol=1e-16)
    # two-level ties
    l = np.zeros(16)
    l[[3, 9, 12]] = 2.0
    l[[1, 14]] = 1.0
    assert list(oracle.topk_sort(l, 5)) == [3, 9, 12, 1, 14]
    assert list(oracle.topk_select(l, 4)) == [3, 9, 12, 1]


def test_topk():
    pin_topk()


def pin_softmax():
    rng = np.random.default_rng(6)
    for _ in range(50):
        E = 256
        l = rng.standard_normal(E) * 3
        k = int(rng.integers(1, 9))
        idx = _lib_topk(l, k)
        w = oracle.softmax_selected(l, idx)
        assert np.allclose(w, softmax(l[idx]), rtol=1e-14, atol=0)
        assert abs(w.sum() - 1.0) < 1e-14
        assert np.allclose(oracle.softmax_selected(l + 7.25, idx), w, rtol=1e-13, atol=0)
        if k == 1:
            assert w[0] == 1.0


def test_softmax():
    pin_softmax()


def pin_silu():
    assert oracle.silu(0.0) == 0.0
    for z in np.linspace(-30, 30, 241):
        assert abs((oracle.silu(z) - oracle.silu(-z)) - z) <= 4e-16 * max(1.0, abs(z))
        assert abs(oracle.silu(z) - z * expit(z)) <= 4e-16 * max(1.0, abs(z))
    assert oracle.silu(800.0) == 800.0
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300


def test_silu():
    pin_silu()


# ------------------------------------------------------------------- union

def _brute_union(idx, E):
    T, k = idx.shape
    ids = sorted(set(int(e) for e in idx.ravel()))
    pairs = []
    for e in ids:
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    pairs.append((t, j))
    offs = [0]
    for e in ids:
        offs.append(offs[-1] + int((idx == e).sum()))
    return ids, offs, pairs


def pin_union():
    rng = np.random.default_rng(7)
    for trial in range(60):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 12))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        if trial % 5 == 0:
            idx[:] = idx[0]
        u = oracle.union(idx, E)
        ids, offs, pairs = _brute_union(idx, E)
        assert u["n_unique"] == len(ids)
        assert list(u["ids"]) == ids
        assert list(u["offsets"]) == offs
        assert [(int(a), int(b)) for a, b in zip(u["pair_token"], u["pair_slot"])] == pairs
        # each (t, j) exactly once, and pair_of is the inverse map
        for p, (t, j) in enumerate(pairs):
            assert u["pair_of"][t * k + j] == p
        assert offs[-1] == T * k
        assert all(a < b for a, b in zip(ids, ids[1:]))
        if trial % 5 == 0:
            assert u["n_unique"] == k


def test_union():
    pin_union()


# ---------------------------------------------------------- expert / layer

def pin_expert_dense():
    rng = np.random.default_rng(8)
    d, f = 256, 128
    blob = _rand_blob(rng, d, f)
    x = rng.standard_normal(d).astype(np.float32).astype(np.float64)
    Wg, Wu, Wd = _dense.dense_expert(blob, d, f)
    o = oracle.expert(blob, d, f, x)
    g, u = Wg @ x, Wu @ x
    h = _dense.silu(g) * u
    y = Wd @ h
    assert np.allclose(o["g"], g, rtol=1e-12, atol=1e-12)
    assert np.allclose(o["u"], u, rtol=1e-12, atol=1e-12)
    assert np.allclose(o["h"], h, rtol=1e-12, atol=1e-12)
    assert np.allclose(o["y"], y, rtol=1e-11, atol=1e-11)
    assert np.allclose(o["yabs"], np.abs(Wd * h[None, :]).sum(axis=1), rtol=1e-12, atol=0)


def test_expert_dense():
    pin_expert_dense()


def pin_onehot_gate():
    """Routing forced to one expert with weight 1 and a zero residual gives
    exactly that expert's dense feed-forward."""
    blobs, R, x = _tiny_inputs()
    xd = x[0].astype(np.float64)
    for e in (0, 7, 15):
        idx = np.array([e, (e + 1) % TINY.E], dtype=np.int32)
        w = np.array([1.0, 0.0])
        out, l1 = oracle.moe_token(xd, TINY.d, TINY.f, {i: blobs[i] for i in range(TINY.E)}, None, idx, w,
                                   np.zeros(TINY.d), TINY.E)
        ref = _dense.dense_ffn(*_dense.dense_expert(blobs[e], TINY.d, TINY.f), xd)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_onehot_gate():
    pin_onehot_gate()


def pin_dense_all_experts():
    """k = E: the sparse layer becomes a dense soft mixture over every expert
    (the same kind of check the pages describe for sparse attention forced to
    select every key; project profile, 'conservative correctness')."""
    blobs, R, x = _tiny_inputs(layer=1)
    shared = synth.expert_blobs(TINY, 1, TINY.E, TINY.E + 1)[0]
    xd = x[0].astype(np.float64)
    k = TINY.E
    l, idx, w = oracle.route_token(R, None, xd, k)
    out, _ = oracle.moe_token(xd, TINY.d, TINY.f, {i: blobs[i] for i in range(TINY.E)}, shared, idx, w, xd,
                              TINY.E)
    ref, sel, wr = _dense.dense_moe_all(blobs, shared, R, None, xd, TINY.d, TINY.f, k)
    assert np.array_equal(np.sort(idx), np.arange(k))
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_dense_all_experts():
    pin_dense_all_experts()


def pin_tiny_layer_bruteforce():
    for layer in (0, 2):
        blobs, R, x = _tiny_inputs(layer)
        xd = x[0].astype(np.float64)
        l, idx, w = oracle.route_token(R, None, xd, TINY.k)
        out, _ = oracle.moe_token(xd, TINY.d, TINY.f, {i: blobs[i] for i in range(TINY.E)}, None, idx, w, xd,
                                  TINY.E)
        ref, sel, wr = _dense.dense_moe_all(blobs, None, R, None, xd, TINY.d, TINY.f, TINY.k)
        assert list(idx) == list(sel)
        assert np.allclose(w, wr, rtol=1e-13, atol=0)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_tiny_layer_bruteforce():
    pin_tiny_layer_bruteforce()


def pin_grouped_layer():
    """The grouped form (each expert dequantised once, fp64 matrix products
    over its tokens) against the per-token definition, which the pins above
    fix: same outputs and L1 norms up to fp64 summation order, on a routing
    with ragged groups, a dropped slot, a shared expert and a separate
    residual."""
    w = synth.Workload(name="grouped_pin", d=192, f=128, E=12, k=3, T=30, n_shared=1, zipf=1.1,
                       seed=synth.BASE_SEED + 77)
    blobs = synth.expert_blobs(w, 0, 0, w.E)
    shared = synth.shared_blob(w, 0)
    X = synth.activations(w, stream=0).astype(np.float64)
    rng = np.random.default_rng(77)
    idx = np.stack([rng.permutation(w.E)[:w.k] for _ in range(w.T)]).astype(np.int32)
    idx[4, 2] = -1
    wts = rng.uniform(0.1, 1.0, size=(w.T, w.k))
    res = rng.normal(size=X.shape)
    ref, ref_l1 = oracle.moe_layer(X, w.d, w.f, {e: blobs[e] for e in range(w.E)}, shared, idx, wts, res, E=w.E)
    out, l1 = oracle.moe_layer_grouped(X, w.d, w.f, lambda e: blobs[e], shared, idx, wts, res, threads=3)
    assert np.all(np.abs(out - ref) <= 1e-12 * ref_l1)
    assert np.allclose(l1, ref_l1, rtol=1e-12, atol=0)


def test_grouped_layer():
    pin_grouped_layer()


def pin_l1_norm():
    blobs, R, x = _tiny_inputs()
    xd = x[0].astype(np.float64)
    l, idx, w = oracle.route_token(R, None, xd, TINY.k)
    out, l1 = oracle.moe_token(xd, TINY.d, TINY.f, {i: blobs[i] for i in range(TINY.E)}, None, idx, w, xd, TINY.E)
    ref = np.abs(xd).copy()
    for j, e in enumerate(idx):
        Wg, Wu, Wd = _dense.dense_expert(blobs[e], TINY.d, TINY.f)
        h = _dense.silu(Wg @ xd) * (Wu @ xd)
        ref += abs(w[j]) * np.abs(Wd * h[None, :]).sum(axis=1)
    assert np.allclose(l1, ref, rtol=1e-12, atol=0)
    assert np.all(l1 >= np.abs(out) * (1 - 1e-12))


def test_l1_norm():
    pin_l1_norm()


def pin_rmsnorm():
    for c in (1.0, -3.5, 1e-4, 250.0):
        r = np.full(6144, c)
        x = oracle.rmsnorm(r, 1e-6)
        assert np.allclose(x, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    r = np.random.default_rng(9).standard_normal(512) * 40
    x1 = oracle.rmsnorm(r, 0.0)
    x2 = oracle.rmsnorm(r * 8.0, 0.0)
    assert np.allclose(x1, x2, rtol=1e-15, atol=0)
    assert abs(np.mean(x1 ** 2) - 1.0) < 1e-14


def test_rmsnorm():
    pin_rmsnorm()


# ------------------------------------------------------ expert top-p

def _topp_reference(l, idx, p):
    """The rule written out with scipy's softmax and numpy sums: the shortest
    prefix of the top-k whose gate weights reach p, then the softmax over it."""
    w = softmax(l[idx])
    m = len(idx)
    if p < 1.0:
        m = 1
        while m < len(idx) and w[:m].sum() < p:
            m += 1
    return m, softmax(l[idx[:m]])


def pin_expert_top_p():
    rng = np.random.default_rng(17)
    E, k = 64, 8
    seen = set()
    for trial in range(40):
        l = rng.standard_normal(E) * (0.5 + trial % 4)
        idx = np.lexsort((np.arange(E), -l))[:k].astype(np.int32)
        w = softmax(l[idx])
        for p in (0.3, 0.5, 0.7, 0.9):
            cums = np.cumsum(w)
            if np.min(np.abs(cums - p)) < 1e-9:
                continue  # a prefix sum at p itself: either side is a valid reading of the boundary
            m, wk = _topp_reference(l, idx, p)
            oi, ow, om = oracle.expert_top_p(l, idx, w, p)
            assert om == m, (trial, p, om, m)
            assert np.array_equal(oi[:m], idx[:m]) and np.all(oi[m:] == -1)
            assert np.allclose(ow[:m], wk, rtol=1e-13, atol=0) and np.all(ow[m:] == 0.0)
            assert abs(ow.sum() - 1.0) < 1e-14
            # the kept mass before the last kept expert is below p, with it at or above
            assert (m == 1 or w[:m - 1].sum() < p) and (m == k or w[:m].sum() >= p)
            seen.add(m)
    assert len(seen) >= 3  # the cases exercise several kept counts
    # p = 1 keeps the whole routing; a tiny p keeps the first expert with weight 1
    l = rng.standard_normal(E)
    idx = np.lexsort((np.arange(E), -l))[:k].astype(np.int32)
    w = softmax(l[idx])
    oi, ow, om = oracle.expert_top_p(l, idx, w, 1.0)
    assert om == k and np.array_equal(oi, idx) and np.allclose(ow, w, rtol=1e-14, atol=0)
    oi, ow, om = oracle.expert_top_p(l, idx, w, 1e-12)
    assert om == 1 and oi[0] == idx[0] and ow[0] == 1.0 and np.all(oi[1:] == -1)


def pin_union_with_dropped_slots():
    rng = np.random.default_rng(5)
    T, E, k = 6, 12, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    keep = rng.integers(1, k + 1, size=T)
    for t in range(T):
        idx[t, keep[t]:] = -1
    u = oracle.union(idx, E)
    # brute force over the kept (token, slot) pairs
    pairs = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k) if idx[t, j] >= 0)
    assert u["n_unique"] == len(set(e for e, _, _ in pairs))
    assert u["offsets"][-1] == len(pairs) == int(keep.sum())
    for p, (e, t, j) in enumerate(pairs):
        assert u["pair_token"][p] == t and u["pair_slot"][p] == j and u["pair_of"][t * k + j] == p
    for t in range(T):
        for j in range(k):
            if idx[t, j] < 0:
                assert u["pair_of"][t * k + j] == -1


def test_expert_top_p():
    pin_expert_top_p()


def test_union_with_dropped_slots():
    pin_union_with_dropped_slots()


def test_dropped_slots_contribute_nothing():
    """A routing with dropped slots gives the layer output of the kept slots alone."""
    blobs, R, x = _tiny_inputs(1)
    ex = {e: blobs[e] for e in range(TINY.E)}
    x = x[0].astype(np.float64)
    idx = np.array([3, 11], dtype=np.int32)
    w = np.array([1.0, 0.0])
    a, _ = oracle.moe_token(x, TINY.d, TINY.f, ex, None, np.array([3, -1], dtype=np.int32), w, x, TINY.E)
    b, _ = oracle.moe_token(x, TINY.d, TINY.f, ex, None, idx[:1], w[:1], x, TINY.E)
    assert np.array_equal(a, b)


# ------------------------------------------------------ int8 container

def pin_int8_container():
    rng = np.random.default_rng(21)
    rows, cols = 4, 256
    q8 = np.arange(rows * cols, dtype=np.int64).astype(np.uint8)  # every byte value
    sc = rng.uniform(0.0003, 0.0012, rows * cols // 64).astype(np.float16).view(np.uint8)
    with oracle.container_bits(8):
        W = oracle.dequant(q8, sc, rows, cols)
        assert np.array_equal(W, _dense.dense_matrix_i8(q8, sc, rows, cols))
        # byte 0x80 is -128 (column 128, group 2), 0x7F is 127 (group 1), 0xFF is -1 (group 3)
        sg = sc.view(np.float16).astype(np.float64)
        assert W[0, 128] == -128 * sg[2] and W[0, 127] == 127 * sg[1] and W[0, 255] == -1 * sg[3]
        d, f = 256, 128
        w8 = synth.WORKLOADS["tiny"].with_(bits=8)
        assert oracle.expert_bytes(d, f) == w8.expert_bytes == 3 * (d * f + d * f // 32)
        blob = synth.expert_blobs(w8, 0, 3, 4)[0]
        x = rng.standard_normal(d).astype(np.float32).astype(np.float64)
        Wg, Wu, Wd = _dense.dense_expert_i8(blob, d, f)
        o = oracle.expert(blob, d, f, x)
        h = _dense.silu(Wg @ x) * (Wu @ x)
        assert np.allclose(o["h"], h, rtol=1e-12, atol=1e-12)
        assert np.allclose(o["y"], Wd @ h, rtol=1e-11, atol=1e-11)
        # a one-hot input picks a column of the gate matrix exactly
        e = np.zeros(d)
        e[37] = 1.0
        assert np.array_equal(oracle.expert(blob, d, f, e)["g"], Wg[:, 37])
    assert oracle.expert_bytes(d, f) == 3 * (d * f // 2 + d * f // 32)  # back to int4 outside


def test_int8_container():
    pin_int8_container()


# -------------------------------------------------------------- page sizes

def _golden_sizes():
    vals = {}
    with open(os.path.join(GOLDEN, "page_sizes.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


def pin_page_sizes():
    g = _golden_sizes()
    be = oracle.expert_bytes(6144, 2048)
    assert be == 20_054_016  # 19.125 MiB per expert at the pages' scale
    assert abs(be / 2 ** 20 - g["expert_mb_approx"]) / g["expert_mb_approx"] < 0.05
    per_token = g["moe_layers"] * g["routed_per_layer"] * be
    assert abs(per_token / 2 ** 30 - g["routed_gb_per_token_approx"]) / g["routed_gb_per_token_approx"] < 0.05
    hot = g["hot_experts"] * be
    assert abs(hot / 2 ** 30 - g["hot_gb_approx"]) / g["hot_gb_approx"] < 0.05
    assert g["group_size"] == 64
    # the blob is three matrices of int4 plus one fp16 scale per 64 weights
    d, f = 6144, 2048
    assert be == 3 * (d * f // 2 + 2 * d * f // 64)
    assert synth.expert_bytes(d, f) == be


def test_page_sizes():
    pin_page_sizes()


# ------------------------------------------------------ planted mistakes

PINS = [pin_nibble_table, pin_dequant_matches_numpy, pin_matvec_closed_forms, pin_router, pin_topk,
        pin_softmax, pin_silu, pin_expert_dense, pin_onehot_gate, pin_dense_all_experts,
        pin_tiny_layer_bruteforce, pin_expert_top_p, pin_grouped_layer]


@pytest.mark.parametrize("name", sorted(_mutants.MUTANTS))
def test_planted_mistakes_are_caught(name):
    with oracle.variant(_mutants.build(name)):
        failed = []
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, "mutant %r passed every pin" % name

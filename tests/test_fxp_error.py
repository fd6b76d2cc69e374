"""Error of the fixed-point activation encoding against plain fp32
dequantisation, per output, on the CPU.

The fixed-point path (COLIMOE_FWD_FXP) encodes every group of 16 activations
v_i as integers X_i = rint(v_i 2^(22-E)) with 2^(E-1) <= max|v| < 2^E and
multiplies them with the int4 weights exactly; the fp32 path ([D] §4
highlight 4: dequantise and multiply in f32) rounds every product q s v to
fp32.  Both then accumulate in fp32.  This test isolates the encoding:
each emulation below applies one path's rounding of the terms and sums the
rounded terms exactly (fp64 accumulation of values that need at most ~60
significant bits is exact up to the final rounding), so the measured
difference to the fp64 oracle is that path's term error alone.

Per output y = sum_i w_i v_i (w_i = q_i s_g) the fixed-point term error is
bounded by
    |dy_fxp| <= 2^-22 sum_g M_g sum_{i in g} |w_i|        (M_g = max_{i in g} |v_i|)
since |v_i - X_i 2^(E-22)| <= 2^(E-23) <= 2^-22 M_g (2^(E-1) <= M_g); plus the
one rounding of each group's exact integer sum to fp32,
    <= 2^-24 (|sum_{i in g} w_i v_i| + 2^-22 M_g sum_{i in g} |w_i|).
The fp32 path's term error is at most 2^-24 sum_i |w_i v_i|.  The test checks
both bounds, and that at the decode shape (d = 6144, f = 2048, N(0,1)
activations for gate/up, SiLU(g) u for down) and at d = f = 16384 the
encoding error of either path stays far inside the acceptance bound
1e-3 (1 + |y|).
"""
import numpy as np
import pytest

import oracle

GROUP = 64  # weights per fp16 scale
FXG = 16    # activations per fixed-point group


def fxp_output(q, s, v):
    """The fixed-point path's terms summed exactly: per 16-group
    float32(V_g) * s_g * 2^(E_g - 22), V_g = sum_i q_i X_i."""
    rows, cols = q.shape
    vg = v.reshape(-1, FXG)
    m = np.abs(vg).max(axis=1)
    E = np.where(m > 0, np.floor(np.log2(np.where(m > 0, m, 1.0))).astype(np.int64) + 1, 0)
    E = np.maximum(E, -100)
    X = np.rint(vg * np.ldexp(1.0, 22 - E)[:, None])
    assert np.all(np.abs(X) <= 2 ** 22)
    V = (q.reshape(rows, -1, FXG) * X[None, :, :]).sum(axis=2)  # exact integers, |V| <= 2^29
    assert np.all(np.abs(V) <= 2 ** 29)
    sg = np.repeat(s, GROUP // FXG, axis=1)  # fp16 scale of each 16-group
    terms = V.astype(np.float32).astype(np.float64) * sg * np.ldexp(1.0, E - 22)[None, :]
    return terms.sum(axis=1), m, E


def fp32_output(q, s, v):
    """The fp32 path's terms summed exactly: fl32(q s) (exact) times fl32(v), rounded to fp32."""
    w = (q * np.repeat(s, GROUP, axis=1)).astype(np.float32)
    prod = (w.astype(np.float64) * v.astype(np.float32).astype(np.float64)).astype(np.float32)
    return prod.astype(np.float64).sum(axis=1)


def _case(rng, rows, cols, v):
    q = rng.integers(-8, 8, size=(rows, cols)).astype(np.float64)
    s = rng.uniform(0.005, 0.02, size=(rows, cols // GROUP)).astype(np.float16).astype(np.float64)
    w = q * np.repeat(s, GROUP, axis=1)
    exact = w @ v  # fp64; each product exact, the sum within cols * 2^-53 of exact
    fx, m, E = fxp_output(q, s, v)
    f32 = fp32_output(q, s, v)
    # bounds
    mg = np.repeat(m, FXG)
    enc_bound = 2.0 ** -22 * (np.abs(w) * mg[None, :]).sum(axis=1)
    vsum = np.abs((w * v[None, :]).reshape(rows, -1, FXG).sum(axis=2))
    round_bound = 2.0 ** -24 * (vsum + 2.0 ** -22 * (np.abs(w) * mg[None, :]).reshape(rows, -1, FXG).sum(axis=2)).sum(axis=1)
    slack = cols * 2.0 ** -52 * np.abs(w * v[None, :]).sum(axis=1)
    assert np.all(np.abs(fx - exact) <= enc_bound + round_bound + slack), "fixed-point term error above its bound"
    assert np.all(np.abs(f32 - exact) <= 2.0 ** -24 * np.abs(w * v[None, :]).sum(axis=1) * 1.0001 + slack)
    acc = 1e-3 * (1.0 + np.abs(exact))
    return dict(fxp=np.abs(fx - exact) / acc, fp32=np.abs(f32 - exact) / acc,
                fxp_rel=np.abs(fx - exact) / np.abs(w * v[None, :]).sum(axis=1),
                fp32_rel=np.abs(f32 - exact) / np.abs(w * v[None, :]).sum(axis=1))


def _silu_h(rng, f):
    g = rng.normal(0, 4.8, f)  # magnitudes of g and u at the decode shape
    u = rng.normal(0, 4.8, f)
    return g / (1 + np.exp(-g)) * u


@pytest.mark.parametrize("d,f,rows", [(6144, 2048, 256), (16384, 16384, 64)], ids=["decode", "max"])
def test_fxp_term_error_within_bound_and_tolerance(d, f, rows):
    rng = np.random.default_rng(d + f)
    x = rng.normal(0, 1, d).astype(np.float32).astype(np.float64)
    gu = _case(rng, rows, d, x)       # gate/up rows: K = d, N(0,1) activations
    h = _silu_h(rng, f).astype(np.float32).astype(np.float64)
    dn = _case(rng, rows, f, h)       # down rows: K = f, heavy-tailed h
    for name, r in (("gate/up", gu), ("down", dn)):
        print("%s d=%d f=%d: encoding error / tolerance max fxp %.2e fp32 %.2e; relative to sum|w v|: "
              "median fxp %.2e fp32 %.2e, max fxp %.2e fp32 %.2e" % (
                  name, d, f, r["fxp"].max(), r["fp32"].max(), np.median(r["fxp_rel"]), np.median(r["fp32_rel"]),
                  r["fxp_rel"].max(), r["fp32_rel"].max()))
        # the encodings' own errors: at most 2% (fixed-point) and 0.5% (fp32
        # products) of the acceptance bound; per term the fixed-point error
        # is about ten times fp32's product rounding, while over a whole
        # output fp32's accumulation roundings (one per product, against one
        # per 16-column group here) dominate both paths' totals
        assert r["fxp"].max() < 2e-2 and r["fp32"].max() < 5e-3
        assert r["fxp_rel"].max() < 2.0 ** -19 and r["fp32_rel"].max() < 2.0 ** -23


def test_fxp_small_elements_keep_relative_precision_per_output():
    """The worst case for the encoding: one large activation per group and the
    rest 2^-10 smaller.  The small elements keep about 12 significant bits
    each, but each output's error stays below 2^-21 of its product L1 norm."""
    rng = np.random.default_rng(7)
    d = 6144
    v = rng.normal(0, 1, d) * 2.0 ** -10
    v[::FXG] = rng.choice([-1.0, 1.0], d // FXG) * 1.5
    v = v.astype(np.float32).astype(np.float64)
    r = _case(rng, 64, d, v)
    print("spiky groups: max fxp error / sum|w v| %.2e, fp32 %.2e" % (r["fxp_rel"].max(), r["fp32_rel"].max()))
    assert r["fxp_rel"].max() < 2.0 ** -21


def test_oracle_agrees_with_the_exact_sum():
    """The emulation's reference is the oracle's own definition: the fp64
    matvec of the dequantised weights (pins the helper against the oracle)."""
    rng = np.random.default_rng(3)
    rows, cols = 8, 256
    q = rng.integers(-8, 8, size=(rows, cols))
    s = rng.uniform(0.005, 0.02, size=(rows, cols // GROUP)).astype(np.float16)
    nib = ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
    v = rng.normal(0, 1, cols)
    y, _ = oracle.matvec(nib.ravel(), s.view(np.uint8).ravel(), rows, cols, v)
    w = q * np.repeat(s.astype(np.float64), GROUP, axis=1)
    assert np.allclose(y, w @ v, rtol=1e-13, atol=1e-13)

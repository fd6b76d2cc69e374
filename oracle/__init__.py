"""CPU oracle of the int4 routed-expert MoE layer (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path; see ``oracle.c`` for what each function computes and the passage of
the colibrì pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """gcc -O2, no fast-math (no reassociation), OpenMP over output rows only."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                               "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _configure(L):
    i32 = ctypes.c_int
    L.oracle_set_bits.argtypes = [i32]
    L.oracle_nibble.restype = i32
    L.oracle_nibble.argtypes = [ctypes.c_uint8, i32]
    L.oracle_half.restype = ctypes.c_double
    L.oracle_half.argtypes = [ctypes.c_uint16]
    L.oracle_weight.restype = ctypes.c_double
    L.oracle_weight.argtypes = [_vp, _vp, i32, i32, i32, i32]
    L.oracle_dequant.argtypes = [_vp, _vp, i32, i32, _vp]
    L.oracle_matvec.argtypes = [_vp, _vp, i32, i32, _vp, _vp, _vp]
    L.oracle_expert_bytes.restype = ctypes.c_size_t
    L.oracle_expert_bytes.argtypes = [i32, i32]
    L.oracle_silu.restype = ctypes.c_double
    L.oracle_silu.argtypes = [ctypes.c_double]
    L.oracle_expert.argtypes = [_vp, i32, i32, _vp, _vp, _vp, _vp, _vp, _vp]
    L.oracle_router.argtypes = [_vp, _vp, _vp, i32, i32, _vp]
    L.oracle_topk_sort.argtypes = [_vp, i32, i32, _vp]
    L.oracle_topk_select.argtypes = [_vp, i32, i32, _vp]
    L.oracle_softmax_selected.argtypes = [_vp, i32, _vp, i32, _vp]
    L.oracle_union.restype = i32
    L.oracle_union.argtypes = [_vp, i32, i32, i32, _vp, _vp, _vp, _vp, _vp]
    L.oracle_rmsnorm.argtypes = [_vp, i32, ctypes.c_double, _vp]
    L.oracle_moe_token.restype = i32
    L.oracle_moe_token.argtypes = [_vp, i32, i32, i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.oracle_route_token.restype = i32
    L.oracle_route_token.argtypes = [_vp, _vp, _vp, i32, i32, i32, _vp, _vp, _vp]
    L.oracle_expert_top_p.argtypes = [_vp, i32, i32, ctypes.c_double, _vp, _vp]
    L.oracle_expert_top_p.restype = i32
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


class variant:
    """Context in which every function below calls another build of the
    oracle's source (a library at ``path`` exporting the same functions).
    The pin-sensitivity test uses it to run the pins against copies of the
    oracle with one mistake planted."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = lib()
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


class container_bits:
    """Context in which the oracle reads int8 (bits=8) or int4 (bits=4) expert containers."""

    def __init__(self, bits: int):
        self.bits = bits

    def __enter__(self):
        lib().oracle_set_bits(self.bits)
        return self

    def __exit__(self, *exc):
        lib().oracle_set_bits(4)


# ------------------------------------------------------------------ pieces

def nibble(byte: int, high: bool) -> int:
    return int(lib().oracle_nibble(byte, 1 if high else 0))


def half(bits: int) -> float:
    return float(lib().oracle_half(bits))


def expert_bytes(d: int, f: int) -> int:
    return int(lib().oracle_expert_bytes(d, f))


def blob_sections(blob: np.ndarray, d: int, f: int, bits: int = 4):
    """(weights, scales) views of gate, up, down in a canonical blob."""
    w = d * f
    nb, ns = (w if bits == 8 else w // 2), (w // 64) * 2
    out, o = [], 0
    for _ in range(3):
        out.append((blob[o:o + nb], blob[o + nb:o + nb + ns]))
        o += nb + ns
    return out


def dequant(nib: np.ndarray, sc: np.ndarray, rows: int, cols: int) -> np.ndarray:
    nib, pn = _c(nib, np.uint8)
    sc, ps = _c(sc, np.uint8)
    W = np.empty((rows, cols), dtype=np.float64)
    lib().oracle_dequant(pn, ps, rows, cols, W.ctypes.data)
    return W


def matvec(nib, sc, rows: int, cols: int, x):
    nib, pn = _c(nib, np.uint8)
    sc, ps = _c(sc, np.uint8)
    x, px = _c(x, np.float64)
    y = np.empty(rows)
    ya = np.empty(rows)
    lib().oracle_matvec(pn, ps, rows, cols, px, y.ctypes.data, ya.ctypes.data)
    return y, ya


def silu(z: float) -> float:
    return float(lib().oracle_silu(z))


def expert(blob: np.ndarray, d: int, f: int, x):
    """One expert: returns dict g, u, h, y, yabs (fp64)."""
    blob, pb = _c(blob, np.uint8)
    x, px = _c(x, np.float64)
    g, u, h = np.empty(f), np.empty(f), np.empty(f)
    y, ya = np.empty(d), np.empty(d)
    lib().oracle_expert(pb, d, f, px, g.ctypes.data, u.ctypes.data, h.ctypes.data, y.ctypes.data, ya.ctypes.data)
    return dict(g=g, u=u, h=h, y=y, yabs=ya)


def router(R: np.ndarray, bias: Optional[np.ndarray], x) -> np.ndarray:
    E, d = R.shape
    R, pR = _c(R, np.float32)
    if bias is not None:
        bias, pb = _c(bias, np.float32)
    else:
        pb = None
    x, px = _c(x, np.float64)
    l = np.empty(E)
    lib().oracle_router(pR, pb, px, E, d, l.ctypes.data)
    return l


def topk_sort(l, k: int) -> np.ndarray:
    l, pl = _c(l, np.float64)
    idx = np.empty(k, dtype=np.int32)
    lib().oracle_topk_sort(pl, l.size, k, idx.ctypes.data)
    return idx


def topk_select(l, k: int) -> np.ndarray:
    l, pl = _c(l, np.float64)
    idx = np.empty(k, dtype=np.int32)
    lib().oracle_topk_select(pl, l.size, k, idx.ctypes.data)
    return idx


def softmax_selected(l, idx) -> np.ndarray:
    l, pl = _c(l, np.float64)
    idx, pi = _c(idx, np.int32)
    w = np.empty(idx.size)
    lib().oracle_softmax_selected(pl, l.size, pi, idx.size, w.ctypes.data)
    return w


def route_token(R, bias, x, k: int):
    """logits, idx, w for one token (top-k by sort, cross-checked by selection)."""
    E, d = R.shape
    R, pR = _c(R, np.float32)
    if bias is not None:
        bias, pb = _c(bias, np.float32)
    else:
        pb = None
    x, px = _c(x, np.float64)
    l = np.empty(E)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k)
    rc = lib().oracle_route_token(pR, pb, px, E, d, k, l.ctypes.data, idx.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle: top-k by sort and by selection disagree")
    return l, idx, w


def expert_top_p(l, idx, w, p: float):
    """Adaptive expert top-p of one token's top-k routing (idx, w in top-k
    order): the shortest prefix whose weight sum reaches p, re-weighted by the
    softmax over the kept logits; dropped entries idx -1, w 0.  Returns
    (idx, w, kept)."""
    l, pl = _c(l, np.float64)
    idx = np.array(idx, dtype=np.int32)
    w = np.array(w, dtype=np.float64)
    m = lib().oracle_expert_top_p(pl, l.size, idx.size, float(p), idx.ctypes.data, w.ctypes.data)
    return idx, w, int(m)


def route(R, bias, X, k: int, top_p: float = 1.0):
    """Route T tokens: logits [T][E], idx [T][k] int32, w [T][k] fp64 (with
    expert top-p when top_p < 1)."""
    X = np.atleast_2d(X)
    T = X.shape[0]
    L = np.empty((T, R.shape[0]))
    I = np.empty((T, k), dtype=np.int32)
    W = np.empty((T, k))
    for t in range(T):
        L[t], I[t], W[t] = route_token(R, bias, X[t].astype(np.float64), k)
        if top_p < 1.0:
            I[t], W[t], _ = expert_top_p(L[t], I[t], W[t], top_p)
    return L, I, W


def union(idx: np.ndarray, E: int):
    """Batch-union lists of a [T][k] routing."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    n = T * k
    ids = np.empty(min(E, n), dtype=np.int32)
    offsets = np.empty(min(E, n) + 1, dtype=np.int32)
    pt, ps, po = (np.empty(n, dtype=np.int32) for _ in range(3))
    nu = lib().oracle_union(idx.ctypes.data, T, k, E, ids.ctypes.data, offsets.ctypes.data, pt.ctypes.data,
                            ps.ctypes.data, po.ctypes.data)
    return dict(n_unique=int(nu), ids=ids[:nu].copy(), offsets=offsets[:nu + 1].copy(), pair_token=pt,
                pair_slot=ps, pair_of=po)


def rmsnorm(r, eps: float = 1e-6) -> np.ndarray:
    r, pr = _c(r, np.float64)
    x = np.empty(r.size)
    lib().oracle_rmsnorm(pr, r.size, eps, x.ctypes.data)
    return x


def moe_token(x, d: int, f: int, experts: Dict[int, np.ndarray], shared: Optional[np.ndarray], idx, w,
              residual, E: int):
    """out, l1 for one token under routing (idx, w); experts maps id -> blob."""
    x, px = _c(x, np.float64)
    idx, pi = _c(idx, np.int32)
    w, pw = _c(w, np.float64)
    residual, prs = _c(residual, np.float64)
    keep = []
    ptrs = (ctypes.c_void_p * E)()
    for e, b in experts.items():
        b = np.ascontiguousarray(b, dtype=np.uint8)
        keep.append(b)
        ptrs[e] = b.ctypes.data
    ps = None
    if shared is not None:
        shared = np.ascontiguousarray(shared, dtype=np.uint8)
        ps = shared.ctypes.data
    out, l1 = np.empty(d), np.empty(d)
    rc = lib().oracle_moe_token(px, d, f, idx.size, ctypes.cast(ptrs, ctypes.c_void_p), ps, pi, pw, prs,
                                out.ctypes.data, l1.ctypes.data)
    if rc != 0:
        raise KeyError("oracle: a selected expert's blob was not supplied")
    return out, l1


def moe_layer(X, d: int, f: int, experts: Dict[int, np.ndarray], shared, idx, w, residual=None, E: int = 0):
    """T tokens through one layer under a given routing.  residual defaults to X."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    R = X if residual is None else np.atleast_2d(np.asarray(residual, dtype=np.float64))
    out = np.empty_like(X)
    l1 = np.empty_like(X)
    for t in range(X.shape[0]):
        out[t], l1[t] = moe_token(X[t], d, f, experts, shared, idx[t], w[t], R[t], E)
    return out, l1


def _dense_expert_rows(blob: np.ndarray, d: int, f: int, Xe: np.ndarray):
    """One expert applied to the m tokens in Xe [m][d]: y [m][d] and
    yabs[t][r] = sum_c |Wd[r][c] h_t[c]|.  The three matrices are decoded once
    by the oracle's own dequantisation (exact q*s in fp64); the products are
    fp64 matrix products (a library routine)."""
    (gn, gs), (un, us), (dn, ds) = blob_sections(blob, d, f)
    Wg = dequant(gn, gs, f, d)
    G = Xe @ Wg.T
    del Wg
    Wu = dequant(un, us, f, d)
    Uu = Xe @ Wu.T
    del Wu
    H = G / (1.0 + np.exp(-G)) * Uu  # SiLU(g) * u, SiLU(z) = z / (1 + e^-z)
    Wd = dequant(dn, ds, d, f)
    Y = H @ Wd.T
    Yabs = np.abs(H) @ np.abs(Wd).T  # |Wd[r][c] h[c]| = |Wd[r][c]| |h[c]|
    return Y, Yabs


def moe_layer_grouped(X, d: int, f: int, blob_of, shared, idx, w, residual=None, threads: int = 0):
    """The same layer as ``moe_layer`` for many tokens, grouped by expert.

    Each distinct expert in idx (and the shared expert) is dequantised once and
    applied to all tokens routed to it with fp64 matrix products, so a
    2048-token prefill-shaped call is checked in seconds instead of minutes.
    out[t] = residual[t] + sum_j w[t][j] y_{idx[t][j]}(x_t) + y_shared(x_t), and
    l1 the per-output L1 norm of the products, exactly as ``moe_token`` defines
    them; only the fp64 summation order differs from its sequential sums.
    blob_of(e) returns expert e's canonical blob; slots with idx -1 add nothing.
    Experts run on ``threads`` worker threads (default: the process's CPUs)."""
    from concurrent.futures import ThreadPoolExecutor
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    T = X.shape[0]
    R = X if residual is None else np.atleast_2d(np.asarray(residual, dtype=np.float64))
    out = R.copy()
    l1 = np.abs(R)
    groups = {}
    for t in range(T):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if e >= 0:
                groups.setdefault(e, []).append((t, j))
    jobs = [(e, groups[e]) for e in sorted(groups)]
    if shared is not None:
        jobs.append((-1, [(t, -1) for t in range(T)]))

    def run(job):
        e, pairs = job
        blob = shared if e < 0 else blob_of(e)
        toks = np.array([t for t, _ in pairs])
        Y, Ya = _dense_expert_rows(np.ascontiguousarray(blob, dtype=np.uint8), d, f, X[toks])
        return e, pairs, Y, Ya

    from threadpoolctl import threadpool_limits
    n = threads or len(os.sched_getaffinity(0))
    # one library thread per worker: the workers already fill the cores
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=max(1, n)) as pool:
        # largest groups first, so the long ones do not start last
        order = sorted(range(len(jobs)), key=lambda i: -len(jobs[i][1]))
        res = dict(zip(order, pool.map(run, [jobs[i] for i in order])))
        for i in range(len(jobs)):
            e, pairs, Y, Ya = res[i]
            for i, (t, j) in enumerate(pairs):
                g = 1.0 if j < 0 else w[t, j]
                out[t] += g * Y[i]
                l1[t] += abs(g) * Ya[i]
    return out, l1

"""colimoe_route_forward_static, the entry point for callers that cannot
allocate: its results must equal colimoe_route_forward's bit for bit (same
kernels, scratch in a fixed device array instead of the caller's workspace),
on two calls in a row with the second one smaller, on a context that has no
workspace at all, without touching a context's own workspace, and a call too
large for the array must be refused with no effect.
"""
import numpy as np
import pytest

import synth
from tests import _parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FXP = 3
# decode-sized experts (fixed-point path, 1 token and batch-union shapes, and
# the fp32 path's one-token pair) on a smaller expert count, and the tiny
# layer (fp32 path)
WIDE = synth.Workload(name="static_wide", d=6144, f=2048, E=32, k=8, T=16, n_shared=1, zipf=1.1, rho=0.6,
                      seed=synth.BASE_SEED + 401)
TINY = synth.WORKLOADS["tiny"]


def _ctx(w, max_tokens, workspace=True):
    import int4_routed_expert_fp32_amd as cm
    from int4_routed_expert_fp32_amd.runtime import MoeContext
    print("context", w.name, w.d, w.f, w.E, w.k, "max_tokens", max_tokens, "workspace", workspace, flush=True)
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=max_tokens)
    if not workspace:  # a context without a workspace: a fresh one, never given one
        bare = cm.colimoe_create(ctx.cfg, ctx.stream.cuda_stream)[1]
        return ctx, bare
    return ctx, None


def _run(fn, ctx_handle, X, with_union, flags):
    """One call of fn (colimoe_route_forward or the static form) on a copy of
    X as input and residual; returns idx, w, residual and the union lists."""
    import int4_routed_expert_fp32_amd as cm
    T, d = X.shape
    x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    res = x.clone()
    k = ctx_handle[1]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    U = ctx_handle[2].new_union(T) if with_union else None
    fn(ctx_handle[0], 0, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(), U.abi() if U is not None else None,
       res.data_ptr(), flags)
    assert cm.colimoe_sync(ctx_handle[0]) == 0
    out = [idx.cpu().numpy(), w.cpu().numpy().view(np.uint32), res.cpu().numpy().view(np.uint32)]
    if U is not None:
        u = U.to_host()
        out += [np.array([u["n_unique"]])] + [u[key] for key in ("ids", "offsets", "pair_token", "pair_slot",
                                                                   "pair_of")]
    return out


@pytest.mark.parametrize("w,flags,sizes", [(WIDE, FXP, (16, 1)), (WIDE, FXP, (5, 2)), (WIDE, 1, (3, 1)),
                                           (TINY, 1, (3, 1))],
                         ids=["wide-16-then-1", "wide-5-then-2", "wide-fp32-3-then-1", "tiny"])
def test_static_matches_route_forward(w, flags, sizes):
    import int4_routed_expert_fp32_amd as cm
    ctx, bare = _ctx(w, max_tokens=max(sizes), workspace=False)
    P.load_layer(ctx, w, 0)
    # the bare context loads the same layer into a buffer of its own
    R, b = synth.router(w, 0), synth.bias(w, 0)
    ex = synth.expert_blobs(w, 0, 0, w.E)
    sh = synth.shared_blob(w, 0) if w.n_shared else None
    buf = torch.empty(ctx.layer_bytes + 256, dtype=torch.uint8, device="cuda")
    dst = buf[(-buf.data_ptr()) % 256:][:ctx.layer_bytes]
    cm.colimoe_load_experts(bare, 0, R.ctypes.data, b.ctypes.data if b is not None else None, ex.ctypes.data,
                            sh.ctypes.data if sh is not None else None, dst.data_ptr(), ctx.layer_bytes)
    for call, T in enumerate(sizes):
        X = synth.activations(w.with_(T=T), stream=50 + call)
        print("call %d: T=%d flags=%d" % (call, T, flags), flush=True)
        for with_union in (True, False):
            ref = _run(cm.colimoe_route_forward, (ctx.ctx, w.k, ctx), X, with_union, flags)
            ws_before = ctx.ws.clone()
            got = _run(cm.colimoe_route_forward_static, (ctx.ctx, w.k, ctx), X, with_union, flags)
            assert torch.equal(ctx.ws, ws_before), "the static call touched the context's workspace"
            got_bare = _run(cm.colimoe_route_forward_static, (bare, w.k, ctx), X, with_union, flags)
            for a, g, gb in zip(ref, got, got_bare):
                assert np.array_equal(a, g), "static call differs from colimoe_route_forward (T=%d)" % T
                assert np.array_equal(a, gb), "static call on a context without workspace differs (T=%d)" % T
    cm.colimoe_destroy(bare)


def test_static_refuses_calls_larger_than_its_array():
    import int4_routed_expert_fp32_amd as cm
    w = WIDE
    T = 80  # this layer's workspace at 80 tokens exceeds 32 MiB
    ctx, _ = _ctx(w, max_tokens=T)
    assert cm.lib().colimoe_workspace_bytes(cm.make_config(w.d, w.f, w.E, w.k, 1, w.n_shared, T)) > \
        cm.COLIMOE_STATIC_SCRATCH_BYTES
    P.load_layer(ctx, w, 0)
    X = synth.activations(w.with_(T=T), stream=60)
    x = torch.from_numpy(X).cuda()
    res = x.clone()
    idx = torch.full((T, w.k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((T, w.k), -7.0, dtype=torch.float32, device="cuda")
    rc = cm.colimoe_route_forward_static(ctx.ctx, 0, x.data_ptr(), T, idx.data_ptr(), wt.data_ptr(), None,
                                         res.data_ptr(), FXP, check=False)
    assert rc == cm.COLIMOE_E_WORKSPACE
    ctx.sync()
    assert torch.equal(res, x) and bool((idx == -7).all()) and bool((wt == -7.0).all())
    # the largest call that fits still runs, and equals the workspace form
    Tmax = max(t for t in range(1, T) if cm.lib().colimoe_workspace_bytes(
        cm.make_config(w.d, w.f, w.E, w.k, 1, w.n_shared, t)) <= cm.COLIMOE_STATIC_SCRATCH_BYTES)
    print("largest static call: T=%d" % Tmax, flush=True)
    Xm = X[:Tmax]
    a = _run(cm.colimoe_route_forward, (ctx.ctx, w.k, ctx), Xm, False, FXP)
    b = _run(cm.colimoe_route_forward_static, (ctx.ctx, w.k, ctx), Xm, False, FXP)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)

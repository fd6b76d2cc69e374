"""Host-side error codes of the C ABI on a live context.

Every status the header lists for a host-side check is provoked here through
the library itself: T outside [0, max_tokens] and a layer index out of range
(E_SHAPE), a layer without weights (E_NOT_LOADED), no workspace or one too
small (E_WORKSPACE), a null, misaligned or wrong-flag argument (E_ARG).  Each
of these calls returns before anything is enqueued; afterwards the context
still works (a routed call on the same stream succeeds and syncs clean).
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module", autouse=True)
def _builds():
    synth.build(force=False)


def _aligned(n_bytes, dev):
    raw = torch.empty(n_bytes + 256, dtype=torch.uint8, device=dev)
    off = (-raw.data_ptr()) % 256
    return raw, raw.data_ptr() + off


def test_error_codes_from_the_host():
    import int4_routed_expert_fp32_amd as cm
    print("abi errors on", W.name, flush=True)
    dev = torch.device("cuda")
    cfg = cm.make_config(W.d, W.f, W.E, W.k, 2, W.n_shared, 4)
    rc, ctx = cm.colimoe_create(cfg, torch.cuda.current_stream(dev).cuda_stream, check=False)
    assert rc == cm.COLIMOE_OK and ctx
    keep = []
    try:
        x = torch.from_numpy(synth.activations(W, 0, 4)).to(dev)
        idx = torch.empty((4, W.k), dtype=torch.int32, device=dev)
        w = torch.empty((4, W.k), dtype=torch.float32, device=dev)
        res = torch.zeros((4, W.d), dtype=torch.float32, device=dev)

        # layer 0 loaded, layer 1 not, no workspace yet
        lb = cm.colimoe_layer_bytes(cfg)
        raw, dst = _aligned(lb, dev)
        keep.append(raw)
        router = np.ascontiguousarray(synth.router(W, 0), dtype=np.float32)
        experts = np.ascontiguousarray(synth.expert_blobs(W, 0, 0, W.E), dtype=np.uint8)
        assert cm.colimoe_load_experts(ctx, 0, router.ctypes.data, None, experts.ctypes.data, None, dst, lb,
                                       check=False) == cm.COLIMOE_OK
        # a layer buffer that is too small or misaligned is refused
        assert cm.colimoe_load_experts(ctx, 1, router.ctypes.data, None, experts.ctypes.data, None, dst, lb - 1,
                                       check=False) != cm.COLIMOE_OK
        assert cm.colimoe_load_experts(ctx, 1, router.ctypes.data, None, experts.ctypes.data, None, dst + 4, lb,
                                       check=False) == cm.COLIMOE_E_ARG

        route = lambda layer, T, xp=x.data_ptr(): cm.colimoe_route(ctx, layer, xp, T, idx.data_ptr(),
                                                                   w.data_ptr(), None, None, check=False)
        assert route(0, 1) == cm.COLIMOE_E_WORKSPACE
        assert route(1, 1) == cm.COLIMOE_E_NOT_LOADED
        assert route(2, 1) == cm.COLIMOE_E_SHAPE
        assert route(-1, 1) == cm.COLIMOE_E_SHAPE
        assert route(0, 5) == cm.COLIMOE_E_SHAPE
        assert route(0, -1) == cm.COLIMOE_E_SHAPE

        wsb = cm.colimoe_workspace_bytes(cfg)
        raw, ws = _aligned(wsb, dev)
        keep.append(raw)
        assert cm.colimoe_set_workspace(ctx, ws, wsb - 1, check=False) == cm.COLIMOE_E_WORKSPACE
        assert cm.colimoe_set_workspace(ctx, ws + 16, wsb, check=False) == cm.COLIMOE_E_ARG
        assert cm.colimoe_set_workspace(ctx, ws, wsb, check=False) == cm.COLIMOE_OK

        # argument checks, all before any launch
        assert route(0, 1, x.data_ptr() + 4) == cm.COLIMOE_E_ARG  # x not 16-byte aligned
        assert cm.colimoe_route(ctx, 0, x.data_ptr(), 1, idx.data_ptr() + 2, w.data_ptr(), None, None,
                                check=False) == cm.COLIMOE_E_ARG
        assert cm.colimoe_route(ctx, 0, 0, 1, idx.data_ptr(), w.data_ptr(), None, None,
                                check=False) == cm.COLIMOE_E_ARG
        fwd = lambda flags, rp=res.data_ptr(): cm.colimoe_forward(ctx, 0, x.data_ptr(), 1, idx.data_ptr(),
                                                                  w.data_ptr(), None, rp, flags, check=False)
        assert fwd(99) == cm.COLIMOE_E_ARG
        assert fwd(cm.COLIMOE_FWD_AUTO, res.data_ptr() + 4) == cm.COLIMOE_E_ARG
        # the fixed-point path needs d and f of at least 2048: refused, not replaced
        assert fwd(cm.COLIMOE_FWD_FXP) == cm.COLIMOE_E_SHAPE
        assert cm.colimoe_rmsnorm_route_forward(ctx, 0, res.data_ptr(), 1, -1.0, x.data_ptr(), idx.data_ptr(),
                                                w.data_ptr(), None, 0, check=False) == cm.COLIMOE_E_ARG
        assert cm.colimoe_sync(ctx, check=False) == cm.COLIMOE_OK

        # the context is intact: a real call goes through
        assert route(0, 4) == cm.COLIMOE_OK
        assert cm.colimoe_sync(ctx, check=False) == cm.COLIMOE_OK
        ids = idx.cpu().numpy()
        assert ((ids >= 0) & (ids < W.E)).all()
        assert all(len(set(r)) == W.k for r in ids.tolist())
    finally:
        cm.colimoe_destroy(ctx)
        torch.cuda.synchronize()

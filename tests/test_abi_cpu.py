"""The C-ABI library loads and exports every symbol include/colimoe.h declares;
host-side validation and size queries answer without touching a GPU."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_fp32_amd as cm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "colimoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(colimoe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_named_calls():
    names = _declared()
    for n in ("colimoe_load_experts", "colimoe_route", "colimoe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = cm.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert sorted(cm.EXPORTED) == _declared()


def test_sizes_match_the_container():
    cfg8 = cm.make_config(6144, 2048, 256, 8, 1, 1, 1, flags=cm.COLIMOE_CFG_INT8)
    assert cm.colimoe_expert_bytes(cfg8) == 3 * 6144 * 2048 * 33 // 32  # int8 weights + fp16 scales per 64
    cfg = cm.make_config(6144, 2048, 256, 8, 1, 1, 1)
    assert cm.colimoe_expert_bytes(cfg) == 20_054_016
    lb = cm.colimoe_layer_bytes(cfg)
    assert lb == 257 * 20_054_016 + 256 * 6144 * 4 + 1024
    assert cm.colimoe_workspace_bytes(cfg) > 0


@pytest.mark.parametrize("bad", [
    dict(d=100), dict(f=96), dict(n_experts=0), dict(n_experts=2000), dict(top_k=0), dict(top_k=17),
    dict(top_k=20, n_experts=16), dict(n_shared=2), dict(group_size=32), dict(max_tokens=0), dict(flags=2),
    dict(n_layers=0), dict(d=32768),
])
def test_invalid_configs_rejected_before_any_gpu_call(bad):
    base = dict(d=256, f=128, n_experts=16, top_k=2, n_layers=1, n_shared=0, max_tokens=1)
    base.update(bad)
    cfg = cm.make_config(**base)
    assert cm.colimoe_expert_bytes(cfg) == 0
    assert cm.colimoe_layer_bytes(cfg) == 0
    assert cm.colimoe_workspace_bytes(cfg) == 0
    rc, ctx = cm.colimoe_create(cfg, None, check=False)
    assert rc == cm.COLIMOE_E_SHAPE and not ctx


def test_null_arguments_rejected():
    L = cm.lib()
    assert L.colimoe_create(None, None, None) == cm.COLIMOE_E_ARG
    assert L.colimoe_route(None, 0, None, 1, None, None, None, None) == cm.COLIMOE_E_ARG
    assert L.colimoe_set_expert_top_p(None, 0.7) == cm.COLIMOE_E_ARG
    assert L.colimoe_forward(None, 0, None, 1, None, None, None, None, 0) == cm.COLIMOE_E_ARG
    assert L.colimoe_load_experts(None, 0, None, None, 0) == cm.COLIMOE_E_ARG
    assert L.colimoe_union_build(None, None, 1, None) == cm.COLIMOE_E_ARG
    assert L.colimoe_sync(None) == cm.COLIMOE_E_ARG
    assert L.colimoe_route_forward(None, 0, None, 1, None, None, None, None, 0) == cm.COLIMOE_E_ARG
    assert L.colimoe_rmsnorm_route_forward(None, 0, None, 1, 1e-6, None, None, None, None, 0) == cm.COLIMOE_E_ARG
    assert L.colimoe_rmsnorm(None, None, 1, 1e-6, None) == cm.COLIMOE_E_ARG
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert cm.status_str(s)

"""Device-buffer bookkeeping over the C ABI, using PyTorch only for memory and streams.

``MoeContext`` allocates the layer buffers and the workspace as torch uint8
tensors on the GPU, loads host arrays through ``colimoe_load_experts`` and
calls ``colimoe_route`` / ``colimoe_forward`` with their data pointers.  All
arithmetic happens in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import (COLIMOE_FWD_AUTO, colimoe_cache_get_info, colimoe_cache_repin, colimoe_cache_set_autorepin,
               colimoe_cache_set_prefetch, colimoe_cache_stats, colimoe_cache_usage, colimoe_cache_usage_load,
               colimoe_cache_usage_save, colimoe_create, colimoe_debug_expert, colimoe_destroy,
               colimoe_expert_cache_bytes, colimoe_forward, colimoe_host_layer_bytes, colimoe_load_experts_host,
               colimoe_set_expert_cache, colimoe_set_expert_top_p,
               colimoe_layer_bytes, colimoe_load_experts, colimoe_rmsnorm, colimoe_rmsnorm_route_forward, colimoe_route,
               colimoe_route_forward,
               colimoe_set_stream,
               colimoe_set_workspace, colimoe_sync, colimoe_union_build, colimoe_workspace_bytes, colimoe_expert_bytes, make_config,
               make_union)


@dataclass
class UnionTensors:
    n_unique: torch.Tensor
    ids: torch.Tensor
    offsets: torch.Tensor
    pair_token: torch.Tensor
    pair_slot: torch.Tensor
    pair_of: torch.Tensor

    def abi(self):
        return make_union(self.n_unique.data_ptr(), self.ids.data_ptr(), self.offsets.data_ptr(),
                          self.pair_token.data_ptr(), self.pair_slot.data_ptr(), self.pair_of.data_ptr())

    def to_host(self) -> Dict[str, np.ndarray]:
        nu = int(self.n_unique.item())
        return dict(n_unique=nu, ids=self.ids[:nu].cpu().numpy(), offsets=self.offsets[:nu + 1].cpu().numpy(),
                    pair_token=self.pair_token.cpu().numpy(), pair_slot=self.pair_slot.cpu().numpy(),
                    pair_of=self.pair_of.cpu().numpy())


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


class MoeContext:
    """One library context with its own workspace and up to n_layers loaded layers."""

    def __init__(self, d: int, f: int, n_experts: int, top_k: int, n_layers: int = 1, n_shared: int = 0,
                 max_tokens: int = 1, device: str = "cuda", stream: Optional[torch.cuda.Stream] = None,
                 cfg_flags: int = 0):
        self.cfg = make_config(d, f, n_experts, top_k, n_layers, n_shared, max_tokens, flags=cfg_flags)
        self.d, self.f, self.E, self.k = d, f, n_experts, top_k
        self.n_layers, self.n_shared, self.max_tokens = n_layers, n_shared, max_tokens
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        _, self.ctx = colimoe_create(self.cfg, self.stream.cuda_stream)
        self.expert_bytes = colimoe_expert_bytes(self.cfg)
        self.layer_bytes = colimoe_layer_bytes(self.cfg)
        self.ws_bytes = colimoe_workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        self._ws_view = self._aligned(self.ws, self.ws_bytes)
        colimoe_set_workspace(self.ctx, self._ws_view.data_ptr(), self.ws_bytes)
        self.layers: Dict[int, torch.Tensor] = {}

    @staticmethod
    def _aligned(t: torch.Tensor, nbytes: int) -> torch.Tensor:
        off = (-t.data_ptr()) % 256
        return t[off:off + nbytes]

    def set_expert_top_p(self, p: float) -> None:
        colimoe_set_expert_top_p(self.ctx, p)

    def set_stream(self, stream: torch.cuda.Stream) -> None:
        self.stream = stream
        colimoe_set_stream(self.ctx, stream.cuda_stream)

    def load_layer(self, layer: int, router: np.ndarray, bias: Optional[np.ndarray], experts: np.ndarray,
                   shared: Optional[np.ndarray]) -> None:
        router = np.ascontiguousarray(router, dtype=np.float32)
        assert router.shape == (self.E, self.d)
        experts = np.ascontiguousarray(experts, dtype=np.uint8)
        assert experts.size == self.E * self.expert_bytes
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            assert bias.shape == (self.E,)
        if shared is not None:
            shared = np.ascontiguousarray(shared, dtype=np.uint8)
            assert shared.size == self.expert_bytes
        if layer in getattr(self, "_host_layers", set()):
            self._host_layers.discard(layer)
            self.layers.pop(layer, None)  # a host-resident layer's buffer holds its router only
        buf = self.layers.get(layer)
        if buf is None:
            raw = torch.empty(self.layer_bytes + 256, dtype=torch.uint8, device=self.device)
            buf = self._aligned(raw, self.layer_bytes)
            self.layers[layer] = buf
            self._keep = getattr(self, "_keep", {})
            self._keep[layer] = raw
        colimoe_load_experts(self.ctx, layer, _ptr(router), _ptr(bias) if bias is not None else None, _ptr(experts),
                             _ptr(shared) if shared is not None else None, buf.data_ptr(), self.layer_bytes)

    def set_expert_cache(self, n_slots: int) -> None:
        """An HBM expert cache of n_slots experts for host-resident layers."""
        nbytes = colimoe_expert_cache_bytes(self.cfg, n_slots)
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        self._cache = raw
        colimoe_set_expert_cache(self.ctx, self._aligned(raw, nbytes).data_ptr(), nbytes)

    def load_layer_host(self, layer: int, router: np.ndarray, bias: Optional[np.ndarray], experts: np.ndarray,
                        shared: Optional[np.ndarray]) -> None:
        """Loads a layer whose routed experts stay in pinned host memory (tiered placement)."""
        router = np.ascontiguousarray(router, dtype=np.float32)
        experts = np.ascontiguousarray(experts, dtype=np.uint8)
        assert router.shape == (self.E, self.d) and experts.size == self.E * self.expert_bytes
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
        if shared is not None:
            shared = np.ascontiguousarray(shared, dtype=np.uint8)
        nbytes = colimoe_host_layer_bytes(self.cfg)
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        self._keep = getattr(self, "_keep", {})
        self._keep[layer] = raw
        self.layers[layer] = self._aligned(raw, nbytes)
        self._host_layers = getattr(self, "_host_layers", set())
        self._host_layers.add(layer)
        colimoe_load_experts_host(self.ctx, layer, _ptr(router), _ptr(bias) if bias is not None else None,
                                  _ptr(experts), _ptr(shared) if shared is not None else None,
                                  self.layers[layer].data_ptr(), nbytes)

    def cache_stats(self):
        return colimoe_cache_stats(self.ctx)

    def cache_repin(self, n: int) -> None:
        colimoe_cache_repin(self.ctx, n)

    def cache_info(self):
        return colimoe_cache_get_info(self.ctx)

    def cache_set_prefetch(self, depth: int) -> None:
        """Prefetch the first `depth` experts of each token's predicted routing (0: off)."""
        colimoe_cache_set_prefetch(self.ctx, depth)

    def cache_set_autorepin(self, every_tokens: int, n: int) -> None:
        colimoe_cache_set_autorepin(self.ctx, every_tokens, n)

    def cache_usage(self, layer: int) -> np.ndarray:
        out = np.zeros(self.E, dtype=np.uint32)
        colimoe_cache_usage(self.ctx, layer, out.ctypes.data)
        return out

    def cache_usage_save(self, path: str) -> None:
        colimoe_cache_usage_save(self.ctx, path)

    def cache_usage_load(self, path: str) -> None:
        colimoe_cache_usage_load(self.ctx, path)

    def new_union(self, T: int) -> UnionTensors:
        tk = T * self.k
        ue = min(self.E, tk)
        i32 = dict(dtype=torch.int32, device=self.device)
        return UnionTensors(torch.zeros(1, **i32), torch.zeros(max(ue, 1), **i32), torch.zeros(ue + 1, **i32),
                            torch.zeros(max(tk, 1), **i32), torch.zeros(max(tk, 1), **i32),
                            torch.zeros(max(tk, 1), **i32))

    def route(self, layer: int, x: torch.Tensor, union: Optional[UnionTensors] = None, want_logits: bool = False):
        T = x.shape[0]
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        logits = torch.empty((T, self.E), dtype=torch.float32, device=self.device) if want_logits else None
        colimoe_route(self.ctx, layer, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                      union.abi() if union is not None else None, logits.data_ptr() if want_logits else None)
        return idx, w, logits

    def union_build(self, idx: torch.Tensor, union: UnionTensors) -> None:
        colimoe_union_build(self.ctx, idx.data_ptr(), idx.shape[0], union.abi())

    def forward(self, layer: int, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                union: Optional[UnionTensors], residual: torch.Tensor, flags: int = COLIMOE_FWD_AUTO) -> None:
        T = x.shape[0]
        colimoe_forward(self.ctx, layer, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                        union.abi() if union is not None else None, residual.data_ptr(), flags)

    def route_forward(self, layer: int, x: torch.Tensor, union: Optional[UnionTensors], residual: torch.Tensor,
                      flags: int = COLIMOE_FWD_AUTO):
        T = x.shape[0]
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        colimoe_route_forward(self.ctx, layer, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                              union.abi() if union is not None else None, residual.data_ptr(), flags)
        return idx, w

    def rmsnorm_route_forward(self, layer: int, r: torch.Tensor, eps: float, x_out: torch.Tensor,
                              union: Optional[UnionTensors], flags: int = COLIMOE_FWD_AUTO):
        """x_out = RMSNorm(r); r += MoE_layer(x_out); returns (idx, w)."""
        T = r.shape[0]
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        colimoe_rmsnorm_route_forward(self.ctx, layer, r.data_ptr(), T, eps, x_out.data_ptr(), idx.data_ptr(),
                                      w.data_ptr(), union.abi() if union is not None else None, flags)
        return idx, w

    def rmsnorm(self, r: torch.Tensor, eps: float, out: torch.Tensor) -> None:
        colimoe_rmsnorm(self.ctx, r.data_ptr(), r.shape[0], eps, out.data_ptr())

    def debug_expert(self, layer: int, e: int, x: torch.Tensor):
        g = torch.empty(self.f, dtype=torch.float32, device=self.device)
        u = torch.empty_like(g)
        h = torch.empty_like(g)
        y = torch.empty(self.d, dtype=torch.float32, device=self.device)
        colimoe_debug_expert(self.ctx, layer, e, x.data_ptr(), g.data_ptr(), u.data_ptr(), h.data_ptr(), y.data_ptr())
        return g, u, h, y

    def sync(self, check: bool = True) -> int:
        return colimoe_sync(self.ctx, check=check)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            colimoe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

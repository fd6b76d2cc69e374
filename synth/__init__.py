"""Seeded synthetic inputs for the int4 routed-expert MoE layer.

Test and benchmark fixture only: it draws numbers and writes them in the
canonical container format (layout in ``synth.c``); it holds none of the
method's arithmetic.  Both the CPU oracle and the HIP library consume these
inputs, each decoding them on its own.

The workloads mirror the shapes the colibrì pages describe (article on
kechuai.cn, §1 "background": 8 of 256 routed experts per layer, int4 experts of
about 19 MB; project profile "conservative correctness": group-size-64 int4
container): synthetic tensors stand in for GLM-5.2 weights, which are not
available.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

SCALE_LO, SCALE_HI = 0.005, 0.02
ROUTER_STD = 0.02
BASE_SEED = 0x434F4C49


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP over experts / rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i32, f64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64]
        L.synth_stream.restype = u64
        L.synth_stream.argtypes = [i32, i32, i32]
        L.synth_expert_bytes.restype = ctypes.c_size_t
        L.synth_expert_bytes.argtypes = [i32, i32]
        L.synth_expert_blob.argtypes = [u64, i32, i32, i32, i32, f64, f64, vp]
        L.synth_expert_blobs.argtypes = [u64, i32, i32, i32, i32, i32, f64, f64, vp]
        L.synth_expert_blobs_i8.argtypes = [u64, i32, i32, i32, i32, i32, f64, f64, vp]
        L.synth_expert_bytes_i8.argtypes = [i32, i32]
        L.synth_expert_bytes_i8.restype = ctypes.c_size_t
        L.synth_router.argtypes = [u64, i32, i32, i32, f64, vp]
        L.synth_zipf_bias.argtypes = [u64, i32, i32, f64, vp]
        L.synth_activations.argtypes = [u64, i32, i32, i32, f64, vp]
        _lib = L
    return _lib


@dataclass(frozen=True)
class Workload:
    """One synthetic MoE workload: shapes plus the input recipe."""
    name: str
    d: int            # hidden size
    f: int            # expert intermediate size
    E: int            # routed experts per layer
    k: int            # experts selected per token
    T: int            # token positions per call
    n_shared: int     # always-on shared experts (0 or 1)
    n_layers: int = 1
    zipf: float = 0.0  # Zipf exponent of the per-layer expert bias (0 = no bias)
    rho: float = 0.0   # pairwise correlation of the T activation rows
    seed: int = BASE_SEED
    bits: int = 4      # expert container: int4 or int8 weights, gs64 fp16 scales

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.d, self.f) if self.bits == 4 else int(lib().synth_expert_bytes_i8(self.d, self.f))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _wl(idx, **kw):
    return Workload(seed=BASE_SEED + idx, **kw)


WORKLOADS = {
    "tiny": _wl(0, name="tiny", d=256, f=128, E=16, k=2, T=1, n_shared=0),
    "decode": _wl(1, name="decode", d=6144, f=2048, E=256, k=8, T=1, n_shared=1),
    "stack32": _wl(2, name="stack32", d=6144, f=2048, E=256, k=8, T=1, n_shared=1, n_layers=32, zipf=1.1),
    "union16": _wl(3, name="union16", d=6144, f=2048, E=256, k=8, T=16, n_shared=1, zipf=1.1, rho=0.6),
    "prefill2048": _wl(4, name="prefill2048", d=6144, f=2048, E=256, k=8, T=2048, n_shared=1, zipf=1.1),
    # multi-position verify: a few draft positions of the batch-union recipe
    "verify4": _wl(5, name="verify4", d=6144, f=2048, E=256, k=8, T=4, n_shared=1, zipf=1.1, rho=0.6),
}


def expert_bytes(d: int, f: int) -> int:
    return int(lib().synth_expert_bytes(d, f))


def expert_blobs(w: Workload, layer: int, e0: int, e1: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Canonical blobs of experts [e0, e1) of `layer` (e == E is the shared expert)."""
    be = w.expert_bytes
    n = (e1 - e0) * be
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.size >= n and out.flags.c_contiguous
    if w.bits == 8:  # int8 weights are 16 times larger: scales 16 times smaller keep the same weight range
        lib().synth_expert_blobs_i8(w.seed, layer, e0, e1, w.d, w.f, SCALE_LO / 16, SCALE_HI / 16, out.ctypes.data)
    else:
        lib().synth_expert_blobs(w.seed, layer, e0, e1, w.d, w.f, SCALE_LO, SCALE_HI, out.ctypes.data)
    return out[:n].reshape(e1 - e0, be) if e1 > e0 else out[:0].reshape(0, be)


def shared_blob(w: Workload, layer: int) -> Optional[np.ndarray]:
    if w.n_shared == 0:
        return None
    return expert_blobs(w, layer, w.E, w.E + 1)[0]


def router(w: Workload, layer: int) -> np.ndarray:
    out = np.empty((w.E, w.d), dtype=np.float32)
    lib().synth_router(w.seed, layer, w.E, w.d, ROUTER_STD, out.ctypes.data)
    return out


def bias(w: Workload, layer: int) -> Optional[np.ndarray]:
    if w.zipf == 0.0:
        return None
    out = np.empty(w.E, dtype=np.float32)
    lib().synth_zipf_bias(w.seed, layer, w.E, w.zipf, out.ctypes.data)
    return out


def activations(w: Workload, stream: int = 0, T: Optional[int] = None) -> np.ndarray:
    T = w.T if T is None else T
    out = np.empty((T, w.d), dtype=np.float32)
    lib().synth_activations(w.seed, stream, T, w.d, w.rho, out.ctypes.data)
    return out


def key(seed: int, stream: int) -> int:
    return int(lib().synth_key(seed, stream))


def u64(key_: int, i: int) -> int:
    return int(lib().synth_u64(key_, i))

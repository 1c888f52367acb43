"""Seeded synthetic inputs for the MoE expert stack.

This module writes input data only: canonical expert blobs (random packed
codes plus bf16 scale/bias words), normally distributed router weights and
activations.  It holds none of the MoE block's arithmetic.  The oracle tests,
the GPU tests, the smoke check and the benchmark all draw their inputs from
here, so both sides of every parity check see the same bytes.

Generator: counter-based SplitMix64 (Steele, Lea & Flood, OOPSLA 2014); see
seedgen.c.  The device twin (seedgen_dev.hip) fills multi-GB arenas in HBM
with bytes identical to the host's.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SO = os.path.join(_HERE, "libseedgen.so")
_DEV_SO = os.path.join(_HERE, "libseedgen_dev.so")

# Expert id used for a layer's shared expert in the generator's keying.
SHARED_ID = 0x7FFFFFFF
# Stream ids inside a (seed, layer, expert) key.
_STREAM_Q, _STREAM_SB, _STREAM_ROUTER, _STREAM_ACT, _STREAM_GAMMA = 0, 1, 2, 3, 4


def build(force: bool = False) -> None:
    """Compile the host generator with gcc and the device twin with hipcc."""
    if force or not os.path.exists(_HOST_SO):
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             os.path.join(_HERE, "seedgen.c"), "-o", _HOST_SO + ".tmp", "-lm"])
        os.replace(_HOST_SO + ".tmp", _HOST_SO)
    if force or not os.path.exists(_DEV_SO):
        subprocess.check_call(
            ["hipcc", "-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             os.path.join(_HERE, "seedgen_dev.hip"), "-o", _DEV_SO + ".tmp"])
        os.replace(_DEV_SO + ".tmp", _DEV_SO)


_host = None
_dev = None


def _lib():
    global _host
    if _host is None:
        if not os.path.exists(_HOST_SO):
            build()
        L = ctypes.CDLL(_HOST_SO)
        u64, i32, f32, vp = ctypes.c_uint64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.sg_key.restype = u64
        L.sg_key.argtypes = [u64, u64, u64, u64]
        L.sg_at.restype = u64
        L.sg_at.argtypes = [u64, u64]
        L.sg_bf16_rne.restype = ctypes.c_uint16
        L.sg_bf16_rne.argtypes = [f32]
        L.sg_fill_words.argtypes = [u64, vp, u64, u64]
        L.sg_fill_sb.argtypes = [u64, vp, u64, u64, f32, f32, f32, f32]
        L.sg_blob_bytes.restype = u64
        L.sg_blob_bytes.argtypes = [i32, i32, i32, i32]
        L.sg_blob.argtypes = [u64, i32, i32, i32, i32, i32, i32, f32, f32, f32, f32, vp]
        L.sg_normal.argtypes = [u64, vp, u64, ctypes.c_double]
        _host = L
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_SO):
            raise RuntimeError(f"device generator not built: {_DEV_SO} (run __graft_entry__.build())")
        L = ctypes.CDLL(_DEV_SO)
        u64, i32, f32, vp = ctypes.c_uint64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.sg_dev_blobs.restype = ctypes.c_int
        L.sg_dev_blobs.argtypes = [u64, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, f32, vp, vp]
        _dev = L
    return _dev


@dataclass(frozen=True)
class Config:
    """One synthetic workload: shapes, distributions and seed."""
    name: str
    D: int            # hidden size
    E: int            # routed experts per layer
    K: int            # experts selected per token
    I: int            # expert intermediate size
    bits: int         # 4 or 2
    group: int = 64
    n_shared: int = 1
    layers: int = 1
    tokens: int = 1   # tokens per step (batch)
    steps: int = 1    # decode steps
    router_sigma: float = 0.02
    s_lo: float = 0.005
    s_hi: float = 0.02
    b_lo: float = -0.1
    b_hi: float = 0.0
    eps: float = 1e-6
    gamma_sigma: float = 0.0  # RMSNorm weight: 1 + N(0, gamma_sigma^2) per element and layer (0: all ones)
    seed: int = 0x5EED0000
    feedback: bool = False   # next step's input = this step's output
    streamed: bool = False
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def blob_bytes(self) -> int:
        return blob_bytes(self.D, self.I, self.bits, self.group)

    def replace(self, **kw) -> "Config":
        d = {k: getattr(self, k) for k in self.__dataclass_fields__}
        d.update(kw)
        return Config(**d)


# The five workloads.  Shapes: hidden 4096, 512 experts, K=4 plus a shared
# expert (hakusoku.com, "モデルアーキテクチャ"; toolarium.ru, "Mixture of
# Experts и почему SSD достаточно"); expert intermediate 1024; 60 layers.
CONFIGS = {
    "tiny": Config("tiny", D=256, E=16, K=2, I=128, bits=4, router_sigma=0.05, seed=0x5EED0000),
    "layer": Config("layer", D=4096, E=512, K=4, I=1024, bits=4, seed=0x5EED0001),
    "stack4": Config("stack4", D=4096, E=512, K=4, I=1024, bits=4, layers=60, steps=128,
                     feedback=True, seed=0x5EED0002),
    "stack2": Config("stack2", D=4096, E=512, K=4, I=1024, bits=2, layers=60, steps=128,
                     feedback=True, seed=0x5EED0003),
    "stack2_b32": Config("stack2_b32", D=4096, E=512, K=4, I=1024, bits=2, layers=60, tokens=32,
                         steps=4, seed=0x5EED0003),
    "streamed4": Config("streamed4", D=4096, E=512, K=4, I=1024, bits=4, layers=60, steps=64,
                        streamed=True, seed=0x5EED0004),
}


def blob_bytes(D: int, I: int, bits: int, group: int) -> int:
    return int(_lib().sg_blob_bytes(D, I, bits, group))


def key(seed: int, layer: int, expert: int, stream: int) -> int:
    return int(_lib().sg_key(seed & 0xFFFFFFFFFFFFFFFF, layer & 0xFFFFFFFFFFFFFFFF,
                             expert & 0xFFFFFFFFFFFFFFFF, stream))


def bf16_rne(x: float) -> int:
    return int(_lib().sg_bf16_rne(x))


def blob(cfg: Config, layer: int, expert: int) -> np.ndarray:
    """Canonical blob of (layer, expert) as uint8; expert SHARED_ID = shared."""
    out = np.empty(cfg.blob_bytes, dtype=np.uint8)
    _lib().sg_blob(cfg.seed, layer, expert, cfg.D, cfg.I, cfg.bits, cfg.group,
                   cfg.s_lo, cfg.s_hi, cfg.b_lo, cfg.b_hi, out.ctypes.data)
    return out


def words(k: int, n: int, w0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    _lib().sg_fill_words(k, out.ctypes.data, w0, n)
    return out


def normal(k: int, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _lib().sg_normal(k, out.ctypes.data, n, sigma)
    return out


def router(cfg: Config, layer: int) -> np.ndarray:
    """Router weights of a layer, fp32 [E][D], N(0, router_sigma^2)."""
    return normal(key(cfg.seed, layer, 0, _STREAM_ROUTER), cfg.E * cfg.D, cfg.router_sigma).reshape(cfg.E, cfg.D)


def activation(cfg: Config, token: int) -> np.ndarray:
    """Input activation of token number `token`, fp32 [D], N(0, 1)."""
    return normal(key(cfg.seed, 0, token, _STREAM_ACT), cfg.D, 1.0)


def activations(cfg: Config, token0: int, n: int) -> np.ndarray:
    return np.stack([activation(cfg, token0 + t) for t in range(n)])


def gamma(cfg: Config, layer: int = 0) -> np.ndarray:
    """RMSNorm weight of a layer, fp32 [D]: all ones (the workloads' value),
    or with cfg.gamma_sigma > 0 the seeded 1 + N(0, gamma_sigma^2), distinct
    per layer, for tests that must tell the layers' weights apart."""
    if cfg.gamma_sigma == 0.0:
        return np.ones(cfg.D, dtype=np.float32)
    g = normal(key(cfg.seed, layer, 0, _STREAM_GAMMA), cfg.D, cfg.gamma_sigma)
    return (np.float32(1.0) + g).astype(np.float32)


def dev_blobs(cfg: Config, layer: int, expert0: int, n: int, dst_ptr: int, stream_ptr: int = 0,
              fixed: bool = False) -> None:
    """Fill n consecutive blobs at device address dst_ptr (asynchronous)."""
    rc = _dev_lib().sg_dev_blobs(cfg.seed, layer, expert0, n, 1 if fixed else 0, cfg.D, cfg.I, cfg.bits,
                                 cfg.group, cfg.s_lo, cfg.s_hi, cfg.b_lo, cfg.b_hi, dst_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"sg_dev_blobs failed: {rc}")

"""Seeded synthetic inputs for the MoE expert-slot layer.

Only input manufacture lives here (random tensors and their stored
encodings, brightness profiles, Zipf routing ids).  Nothing in this package
routes, manages a cache or evaluates an expert: the CPU oracle and the GPU
path both consume the bytes produced here and nothing else from it.

The workload shapes follow the five layer configurations of the task
statement: a tiny fp32 layer; a Qwen3-30B-A3B-shaped bf16 decode layer
(128 experts, top-8, hidden 2048, expert intermediate 768); the same layer in
W8A8 under Zipf(0.8) routing; a 48-layer stack of 512-expert top-10 layers
(hidden 2048, intermediate 512) with 4-bit blocks; and a 288-expert bf16
prefill layer (hidden 4096, intermediate 1536, 2048 tokens).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SYNTH_LIB points the wrapper at another build of synth.c (the
# sanitized build the CPU tests load).
_SO = os.environ.get("MOE_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

# tensor tags for the counter-based streams
TAG_X, TAG_G, TAG_WG, TAG_WU, TAG_WD = 1, 2, 3, 4, 5
TAG_B, TAG_ZIPF_PERM, TAG_ZIPF_DRAW, TAG_WARM = 6, 7, 8, 9

# stored weight formats (same codes as the C ABI)
W_F32, W_BF16, W_W8A8, W_Q4B32 = 0, 1, 2, 3
X_F32, X_BF16 = 0, 1

BASE_SEED = 0xE5510000

CONFIGS = {
    "c1": dict(name="tiny-fp32", E=8, k=2, H=64, I=128, T=16, w_type=W_F32, x_dtype=X_F32,
               sigma_w=0.02, sigma_g=0.1, S=4, policy="static", resident=[0, 1, 2, 3], layers=1),
    "c2": dict(name="qwen3-30b-a3b-shaped-bf16-decode", E=128, k=8, H=2048, I=768, T=64, batches=[1, 8, 64],
               w_type=W_BF16, x_dtype=X_BF16, sigma_w=0.02, sigma_g=0.05, S=64, policy="static", layers=1),
    "c3": dict(name="qwen3-30b-a3b-shaped-w8a8-dynamic", E=128, k=8, H=2048, I=768, T=16, steps=256,
               w_type=W_W8A8, x_dtype=X_BF16, sigma_w=0.02, sigma_g=0.05, S=32, policy="lru", zipf_s=0.8,
               layers=1),
    "c4": dict(name="48x512-top10-q4b32-graded-bias", E=512, k=10, H=2048, I=512, T=32, batches=[1, 32],
               w_type=W_Q4B32, x_dtype=X_BF16, sigma_w=0.02, sigma_g=0.05, S=192, policy="static", layers=48,
               cap=-1.0, alpha=0.3),
    "c5": dict(name="288-expert-bf16-prefill", E=288, k=8, H=4096, I=1536, T=2048, w_type=W_BF16,
               x_dtype=X_BF16, sigma_w=0.02, sigma_g=0.05, S=288, S_variant=144, policy="static", layers=1),
}


def config_seed(name: str) -> int:
    return BASE_SEED + int(name[1:])


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (input manufacture only)."""
    if os.environ.get("MOE_SYNTH_LIB"):
        return _SO
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-mf16c", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_normal.restype = i32
        L.synth_normal.argtypes = [u64, i64, dbl, i32, vp, i32]
        L.synth_slab_bytes.restype = i64
        L.synth_slab_bytes.argtypes = [i32, i32, i32]
        L.synth_slabs.restype = i32
        L.synth_slabs.argtypes = [i32, u64, i32, i32, i32, i32, i32, dbl, vp, i64, i32]
        L.synth_encode_slab.restype = i32
        L.synth_encode_slab.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.synth_dirichlet.restype = i32
        L.synth_dirichlet.argtypes = [u64, i32, dbl, vp]
        L.synth_zipf_ids.restype = i32
        L.synth_zipf_ids.argtypes = [u64, u64, i32, i32, i32, dbl, vp]
        _lib = L
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def key(base: int, tag: int, layer: int = 0, expert: int = 0) -> int:
    return int(lib().synth_key(base, tag, layer, expert))


def normal(k: int, shape, sigma: float, dtype: int) -> np.ndarray:
    """N(0, sigma^2) draws of stream k; fp32 array, or bf16 bit patterns (uint16)."""
    n = int(np.prod(shape))
    out = np.empty(shape, dtype=np.float32 if dtype == X_F32 else np.uint16)
    rc = lib().synth_normal(k, n, sigma, dtype, out.ctypes.data, _threads())
    assert rc == 0
    return out


def slab_bytes(w_type: int, H: int, I: int) -> int:
    return int(lib().synth_slab_bytes(w_type, H, I))


def slabs_into(ptr: int, w_type: int, base: int, layer: int, e0: int, e1: int, H: int, I: int, sigma: float,
               slab: int) -> None:
    """Write slabs of experts [e0, e1) to raw memory at ptr (e.g. pinned host)."""
    rc = lib().synth_slabs(w_type, base, layer, e0, e1, H, I, sigma, ptr, slab, _threads())
    if rc != 0:
        raise ValueError(f"synth_slabs failed ({rc})")


def slabs(w_type: int, base: int, layer: int, e0: int, e1: int, H: int, I: int, sigma: float) -> np.ndarray:
    sb = slab_bytes(w_type, H, I)
    out = np.empty((e1 - e0, sb), dtype=np.uint8)
    slabs_into(out.ctypes.data, w_type, base, layer, e0, e1, H, I, sigma, sb)
    return out


def encode_slab(w_type: int, H: int, I: int, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Encode float matrices Wg[I][H], Wu[I][H], Wd[H][I] into one slab."""
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    wu = np.ascontiguousarray(wu, dtype=np.float32)
    wd = np.ascontiguousarray(wd, dtype=np.float32)
    assert wg.shape == (I, H) and wu.shape == (I, H) and wd.shape == (H, I)
    out = np.zeros(slab_bytes(w_type, H, I), dtype=np.uint8)
    rc = lib().synth_encode_slab(w_type, H, I, wg.ctypes.data, wu.ctypes.data, wd.ctypes.data, out.ctypes.data)
    assert rc == 0, rc
    return out


def dirichlet(k: int, E: int, alpha: float) -> np.ndarray:
    out = np.empty(E, dtype=np.float64)
    assert lib().synth_dirichlet(k, E, alpha, out.ctypes.data) == 0
    return out


def zipf_ids(key_perm: int, key_draw: int, T: int, E: int, k: int, s: float) -> np.ndarray:
    out = np.empty((T, k), dtype=np.int32)
    assert lib().synth_zipf_ids(key_perm, key_draw, T, E, k, s, out.ctypes.data) == 0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns (round to nearest even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


# ------------------------------------------------------------ layer inputs


class LayerInputs:
    """All host-side inputs of one MoE layer of a configuration."""

    def __init__(self, cfg: str, layer: int = 0, T: int | None = None, step: int = 0, with_store: bool = True,
                 E: int | None = None):
        c = CONFIGS[cfg]
        self.cfg, self.c = cfg, c
        self.base = config_seed(cfg)
        self.layer = layer
        self.E = E or c["E"]
        self.k, self.H, self.I = c["k"], c["H"], c["I"]
        self.T = T if T is not None else c["T"]
        self.w_type, self.x_dtype = c["w_type"], c["x_dtype"]
        self.slab = slab_bytes(self.w_type, self.H, self.I)
        # activations: a fresh batch per (layer, step); expert index slot carries the step
        self.x = normal(key(self.base, TAG_X, layer, step), (self.T, self.H), 1.0, self.x_dtype)
        # router gate, one row per expert ([out][in] like every weight)
        self.G = normal(key(self.base, TAG_G, layer, 0), (self.E, self.H), c["sigma_g"], self.x_dtype)
        self.store = slabs(self.w_type, self.base, layer, 0, self.E, self.H, self.I, c["sigma_w"]) if with_store else None

    def x_f32(self) -> np.ndarray:
        return self.x if self.x_dtype == X_F32 else bf16_to_f32(self.x)

    def G_f32(self) -> np.ndarray:
        return self.G if self.x_dtype == X_F32 else bf16_to_f32(self.G)

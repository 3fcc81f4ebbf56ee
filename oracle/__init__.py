"""CPU oracle for the MoE expert-slot layer -- TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It wraps ``liboracle.so`` (plain single-threaded C,
see oracle.c) with numpy marshalling; it never touches the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB points the wrapper at another build of oracle.c (the
# mutation test loads copies with planted mistakes this way).
_SO = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

STATIC, LRU, LFU = 0, 1, 2
POLICIES = {"static": STATIC, "lru": LRU, "lfu": LFU}


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc: no fast-math, no FMA contraction."""
    if os.environ.get("MOE_ORACLE_LIB"):
        return _SO
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.oracle_slab_bytes.restype = i64
        L.oracle_slab_bytes.argtypes = [i32, i32, i32]
        L.oracle_decode_expert.argtypes = [i32, vp, i32, i32, vp, vp, vp]
        L.oracle_logits.argtypes = [vp, i32, vp, i32, i32, i32, vp]
        L.oracle_bias_table.argtypes = [vp, i32, i32, f32, vp]
        L.oracle_topk.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_route_weights.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_bias_flat.argtypes = [vp, i32, i32, f32, vp]
        L.oracle_bias_affinity.argtypes = [vp, vp, i32, f32, vp]
        L.oracle_route_weights_damped.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_expert.argtypes = [i32, vp, i32, i32, vp, i32, vp]
        L.oracle_layer.argtypes = [i32, vp, i64, i32, i32, i32, vp, i32, vp, vp, vp, i32, i32, vp, vp, vp]
        L.oracle_manage.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_gather.argtypes = [vp, i32, vp, vp, i64]
        L.oracle_pick_static.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_repick.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_residual.argtypes = [vp, i32, vp, i32, i32, vp]
        for f in ("oracle_decode_expert", "oracle_logits", "oracle_bias_table", "oracle_topk",
                  "oracle_route_weights", "oracle_expert", "oracle_layer", "oracle_manage", "oracle_gather",
                  "oracle_pick_static", "oracle_residual", "oracle_bias_flat", "oracle_bias_affinity",
                  "oracle_route_weights_damped", "oracle_repick"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed ({rc})")


def slab_bytes(w_type, H, I):
    return int(lib().oracle_slab_bytes(w_type, H, I))


def decode_expert(w_type, slab, H, I):
    slab = _c(slab, np.uint8)
    wg = np.empty((I, H), np.float32)
    wu = np.empty((I, H), np.float32)
    wd = np.empty((H, I), np.float32)
    _check(lib().oracle_decode_expert(w_type, _p(slab), H, I, _p(wg), _p(wu), _p(wd)), "decode_expert")
    return wg, wu, wd


def _xarr(x, x_dtype):
    return _c(x, np.float32 if x_dtype == 0 else np.uint16)


def logits(x, x_dtype, G):
    x = _xarr(x, x_dtype)
    G = _xarr(G, x_dtype)
    T, H = x.shape
    E = G.shape[0]
    assert G.shape == (E, H)
    z = np.empty((T, E), np.float32)
    _check(lib().oracle_logits(_p(x), x_dtype, _p(G), T, H, E, _p(z)), "logits")
    return z


def bias_table(b, n_hot, cap):
    b = _c(b, np.float64)
    out = np.empty(b.shape[0], np.float32)
    _check(lib().oracle_bias_table(_p(b), b.shape[0], n_hot, cap, _p(out)), "bias_table")
    return out


def topk(z, k, bias=None):
    z = _c(z, np.float32)
    T, E = z.shape
    ids = np.empty((T, k), np.int32)
    bias = None if bias is None else _c(bias, np.float32)
    _check(lib().oracle_topk(_p(z), _p(bias), T, E, k, _p(ids)), "topk")
    return ids


def route_weights(z, ids):
    z = _c(z, np.float32)
    ids = _c(ids, np.int32)
    T, E = z.shape
    k = ids.shape[1]
    w = np.empty((T, k), np.float32)
    _check(lib().oracle_route_weights(_p(z), _p(ids), T, E, k, _p(w)), "route_weights")
    return w


def bias_flat(b, n_hot, value):
    """0 for the n_hot brightest experts, `value` for every other (-inf: hard mask)."""
    b = _c(b, np.float64)
    out = np.empty(b.shape[0], np.float32)
    _check(lib().oracle_bias_flat(_p(b), b.shape[0], n_hot, value, _p(out)), "bias_flat")
    return out


def bias_affinity(e2s, lam, base=None):
    """base (or 0) plus lam for every expert with e2s[e] >= 0, one fp32 add."""
    e2s = _c(e2s, np.int32)
    base = None if base is None else _c(base, np.float32)
    out = np.empty(e2s.shape[0], np.float32)
    _check(lib().oracle_bias_affinity(_p(e2s), _p(base), e2s.shape[0], lam, _p(out)), "bias_affinity")
    return out


def route_weights_damped(z, bias, ids):
    """Softmax of the biased scores fl32(z + bias) over the picks."""
    z = _c(z, np.float32)
    ids = _c(ids, np.int32)
    bias = None if bias is None else _c(bias, np.float32)
    T, E = z.shape
    k = ids.shape[1]
    w = np.empty((T, k), np.float32)
    _check(lib().oracle_route_weights_damped(_p(z), _p(bias), _p(ids), T, E, k, _p(w)), "route_weights_damped")
    return w


def expert(w_type, slab, H, I, x_row, x_dtype):
    slab = _c(slab, np.uint8)
    x_row = _xarr(x_row, x_dtype)
    o = np.empty(H, np.float64)
    _check(lib().oracle_expert(w_type, _p(slab), H, I, _p(x_row), x_dtype, _p(o)), "expert")
    return o


def layer(w_type, store, E, H, I, x, x_dtype, ids, w, slot_ids=None):
    """Returns (y_full, y_gpu, y_host); the last two are None without slot_ids."""
    store = _c(store, np.uint8).reshape(E, -1)
    x = _xarr(x, x_dtype)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, k = ids.shape
    yf = np.empty((T, H), np.float32)
    yg = np.empty((T, H), np.float32) if slot_ids is not None else None
    yh = np.empty((T, H), np.float32) if slot_ids is not None else None
    sl = None if slot_ids is None else _c(slot_ids, np.int32)
    _check(lib().oracle_layer(w_type, _p(store), store.shape[1], E, H, I, _p(x), x_dtype, _p(ids), _p(sl), _p(w), T,
                              k, _p(yf), _p(yg), _p(yh)), "layer")
    return yf, yg, yh


class Cache:
    """Host-side cache state driven by oracle_manage."""

    def __init__(self, E, S, policy, resident=None):
        self.E, self.S, self.policy = E, S, POLICIES.get(policy, policy)
        self.e2s = np.full(E, -1, np.int32)
        self.s2e = np.full(max(S, 0), -1, np.int32)
        self.last = np.zeros(max(S, 0), np.uint32)
        self.freq = np.zeros(max(S, 0), np.uint32)
        self.step = np.zeros(1, np.uint32)
        if resident is not None:
            for s, e in enumerate(resident):
                self.s2e[s] = e
                self.e2s[e] = s

    def manage(self, ids):
        ids = _c(ids, np.int32).reshape(-1)
        n = ids.shape[0]
        slot_ids = np.empty(n, np.int32)
        miss = np.empty(2 * max(self.S, 1), np.int32)
        host = np.empty(self.E, np.int32)
        n_miss = np.zeros(1, np.int32)
        n_host = np.zeros(1, np.int32)
        stats = np.zeros(4, np.int32)
        _check(lib().oracle_manage(self.policy, self.E, self.S, _p(self.e2s), _p(self.s2e), _p(self.last),
                                   _p(self.freq), _p(self.step), _p(ids), n, _p(slot_ids), _p(miss), _p(n_miss),
                                   _p(host), _p(n_host), _p(stats)), "manage")
        nm, nh = int(n_miss[0]), int(n_host[0])
        return dict(slot_ids=slot_ids, miss=miss[:2 * nm].reshape(nm, 2), host_miss=host[:nh], stats=stats)

    def repick(self, want):
        """Swap the resident set to the distinct valid experts of want (oracle_repick);
        returns the (expert, slot) loads."""
        want = _c(want, np.int32).reshape(-1)
        assert want.shape[0] == self.S
        miss = np.empty(2 * max(self.S, 1), np.int32)
        n_miss = np.zeros(1, np.int32)
        _check(lib().oracle_repick(self.E, self.S, _p(self.e2s), _p(self.s2e), _p(self.last), _p(self.freq),
                                   _p(self.step), _p(want), _p(miss), _p(n_miss)), "repick")
        return miss[:2 * int(n_miss[0])].reshape(-1, 2).copy()


def gather(miss, host_store, slot_store):
    miss = _c(miss, np.int32).reshape(-1)
    assert host_store.flags.c_contiguous and slot_store.flags.c_contiguous
    sb = host_store.shape[1]
    _check(lib().oracle_gather(_p(miss), miss.shape[0] // 2, _p(host_store), _p(slot_store), sb), "gather")


def pick_static(ids, E, S):
    ids = _c(ids, np.int32).reshape(-1)
    out = np.empty(S, np.int32)
    _check(lib().oracle_pick_static(_p(ids), ids.shape[0], E, S, _p(out)), "pick_static")
    return out


def residual(x, x_dtype, y):
    """Next layer's input: bf16(x + y) (bit patterns) for bf16 streams, x + y for fp32."""
    x = _xarr(x, x_dtype)
    y = _c(y, np.float32)
    T, H = x.shape
    out = np.empty_like(x)
    _check(lib().oracle_residual(_p(x), x_dtype, _p(y), T, H, _p(out)), "residual")
    return out

"""Python binding of libmoeslot.so, the gfx950 expert-slot MoE layer.

Argument marshalling only: every function here has the name and argument
order of its C entry point in include/moe_slot.h, takes torch tensors (or
raw integer addresses) for pointers and defaults the stream to torch's
current stream.  All arithmetic runs in the library's HIP kernels (and, for
``moe_ffn_host_misses``, its C++ host pass).  If the library is missing the
import of any function fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SLOT_LIB points the binding at another build of the same sources (the
# host-sanitized build that the CPU tests load); by default, the in-tree one.
_LIB_DEFAULT = os.path.join(_HERE, "lib", "libmoeslot.so")
LIB_PATH = os.environ.get("MOE_SLOT_LIB") or _LIB_DEFAULT

MOE_OK = 0
MOE_E_ARG, MOE_E_ALIGN, MOE_E_DTYPE, MOE_E_SHAPE, MOE_E_HIP, MOE_E_NOMEM = -1, -2, -3, -4, -5, -6
MOE_X_F32, MOE_X_BF16 = 0, 1
MOE_W_F32, MOE_W_BF16, MOE_W_W8A8, MOE_W_Q4B32 = 0, 1, 2, 3
MOE_STATIC, MOE_LRU, MOE_LFU = 0, 1, 2
MOE_MAX_E, MOE_MAX_S, MOE_MAX_K = 4096, 1024, 32
MOE_ROUTE_DAMPED = 1
POLICIES = {"static": MOE_STATIC, "lru": MOE_LRU, "lfu": MOE_LFU}


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, reason: str):
        super().__init__(f"{fn} failed ({code}): {reason}")
        self.code = code


class CacheState(ctypes.Structure):
    _fields_ = [("e2s", ctypes.c_void_p), ("s2e", ctypes.c_void_p), ("last", ctypes.c_void_p),
                ("freq", ctypes.c_void_p), ("step", ctypes.c_void_p), ("E", ctypes.c_int32), ("S", ctypes.c_int32)]


class SlabLayout(ctypes.Structure):
    _fields_ = [("w", ctypes.c_int64 * 3), ("s", ctypes.c_int64 * 3), ("total", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    """moe_layer_desc: one layer as the native step driver sees it."""
    _fields_ = [("G", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("state", CacheState), ("policy", ctypes.c_int),
                ("slot_store", ctypes.c_void_p), ("host_store", ctypes.c_void_p), ("slab_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() (hipcc for gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        sig = {
            "moe_abi_version": (i32, []),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_slab_layout": (i32, [i32, i32, i32, ctypes.POINTER(SlabLayout)]),
            "moe_bias_table": (i32, [vp, i32, i32, f32, vp, vp]),
            "moe_bias_flat": (i32, [vp, i32, i32, f32, vp, vp]),
            "moe_bias_affinity": (i32, [vp, vp, i32, f32, vp, vp]),
            "moe_route": (i32, [vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]),
            "moe_route_ex": (i32, [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
            "cache_init": (i32, [ctypes.POINTER(CacheState), vp, vp]),
            "cache_pick_static": (i32, [vp, i32, i32, i32, vp, vp]),
            "cache_manage": (i32, [ctypes.POINTER(CacheState), i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]),
            "cache_gather": (i32, [vp, vp, i32, vp, vp, sz, vp]),
            "cache_repick": (i32, [ctypes.POINTER(CacheState), vp, vp, vp, vp]),
            "cache_manage_gather": (i32, [ctypes.POINTER(CacheState), i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          sz, vp, i32, vp, vp, vp, vp, vp]),
            "moe_ffn_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
            "moe_ffn_slots": (i32, [vp, i32, vp, vp, i32, i32, vp, sz, i32, i32, i32, i32, vp, vp, sz, vp]),
            "moe_ffn_slots_noalloc": (i32, [vp, i32, vp, vp, i32, i32, vp, sz, i32, i32, i32, i32, vp, vp]),
            "moe_ffn_noalloc_scratch_bytes": (sz, []),
            "moe_ffn_host_misses": (i32, [vp, i32, vp, vp, vp, i32, i32, vp, sz, i32, i32, i32, i32, vp, i32]),
            "moe_combine": (i32, [vp, vp, i32, i32, vp]),
            "moe_residual": (i32, [vp, i32, vp, vp, i32, i32, vp]),
            "moe_step_create": (vp, [i32, i32, i32, i32, i32, i32, i32]),
            "moe_step_destroy": (None, [vp]),
            "moe_step_output": (vp, [vp]),
            "moe_step_stats": (i32, [vp, ctypes.POINTER(ctypes.c_int64), i32]),
            "moe_layer_step": (i32, [vp, ctypes.POINTER(LayerDesc), vp, i32, vp, i32, i32, vp, vp, vp, vp]),
            "moe_stack_step": (i32, [vp, ctypes.POINTER(LayerDesc), i32, vp, i32, i32, i32, vp, vp, vp, vp]),
            "moe_step_set_stream_threshold": (i32, [vp, i32]),
            "moe_step_last_host_mode": (i32, [vp]),
            "moe_fused_spin_limit": (ctypes.c_int64, [ctypes.c_int64]),
            "moe_host_alloc": (vp, [sz]),
            "moe_host_free": (i32, [vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _p(a):
    """Pointer of a tensor / numpy array / int / None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    if hasattr(a, "ctypes"):
        return a.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(a)!r}")


def _stream(s):
    if s is not None:
        return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(name, rc):
    if rc != MOE_OK:
        raise MoeError(name, rc, (lib().moe_last_error() or b"").decode())
    return rc


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_last_error() -> str:
    return (lib().moe_last_error() or b"").decode()


def moe_slab_layout(w_type, H, I) -> SlabLayout:
    out = SlabLayout()
    _check("moe_slab_layout", lib().moe_slab_layout(w_type, H, I, ctypes.byref(out)))
    return out


def moe_bias_table(b, E, n_hot, cap, bias, stream=None):
    return _check("moe_bias_table", lib().moe_bias_table(_p(b), E, n_hot, cap, _p(bias), _stream(stream)))


def moe_route(x, x_dtype, G, bias, ids_in, T, H, E, k, ids, w, logits, stream=None):
    return _check("moe_route", lib().moe_route(_p(x), x_dtype, _p(G), _p(bias), _p(ids_in), T, H, E, k, _p(ids),
                                               _p(w), _p(logits), _stream(stream)))


def moe_route_ex(x, x_dtype, G, bias, ids_in, T, H, E, k, flags, ids, w, logits, stream=None):
    return _check("moe_route_ex", lib().moe_route_ex(_p(x), x_dtype, _p(G), _p(bias), _p(ids_in), T, H, E, k, flags,
                                                     _p(ids), _p(w), _p(logits), _stream(stream)))


def moe_bias_flat(b, E, n_hot, value, bias, stream=None):
    return _check("moe_bias_flat", lib().moe_bias_flat(_p(b), E, n_hot, value, _p(bias), _stream(stream)))


def moe_bias_affinity(e2s, base, E, lam, bias, stream=None):
    return _check("moe_bias_affinity", lib().moe_bias_affinity(_p(e2s), _p(base), E, lam, _p(bias), _stream(stream)))


def cache_state(e2s, s2e, last, freq, step, E, S) -> CacheState:
    return CacheState(_p(e2s), _p(s2e), _p(last), _p(freq), _p(step), E, S)


def cache_init(st, resident, stream=None):
    return _check("cache_init", lib().cache_init(ctypes.byref(st), _p(resident), _stream(stream)))


def cache_pick_static(ids, n_ids, E, S, resident, stream=None):
    return _check("cache_pick_static", lib().cache_pick_static(_p(ids), n_ids, E, S, _p(resident), _stream(stream)))


def cache_manage(st, policy, ids, n_ids, slot_ids, miss, n_miss, host_miss, n_host, stats=None, stream=None):
    return _check("cache_manage", lib().cache_manage(ctypes.byref(st), policy, _p(ids), n_ids, _p(slot_ids), _p(miss),
                                                     _p(n_miss), _p(host_miss), _p(n_host), _p(stats),
                                                     _stream(stream)))


class Doorbell(ctypes.Structure):
    """moe_doorbell: written by cache_manage_gather into pinned host memory, seq last."""
    _fields_ = [("seq", ctypes.c_int32), ("n_miss", ctypes.c_int32), ("n_host", ctypes.c_int32),
                ("stats", ctypes.c_int32 * 4), ("err", ctypes.c_int32)]


def cache_manage_gather(st, policy, ids, n_ids, w, slot_ids, miss, n_miss, host_miss, n_host, stats, host_store,
                        slot_store, slab_bytes, sync, seq, bell=None, bell_ids=None, bell_slots=None, bell_w=None,
                        stream=None):
    return _check("cache_manage_gather",
                  lib().cache_manage_gather(ctypes.byref(st), policy, _p(ids), n_ids, _p(w), _p(slot_ids), _p(miss),
                                            _p(n_miss), _p(host_miss), _p(n_host), _p(stats), _p(host_store),
                                            _p(slot_store), slab_bytes, _p(sync), seq, _p(bell), _p(bell_ids),
                                            _p(bell_slots), _p(bell_w), _stream(stream)))


def cache_repick(st, want, miss, n_miss, stream=None):
    return _check("cache_repick", lib().cache_repick(ctypes.byref(st), _p(want), _p(miss), _p(n_miss),
                                                     _stream(stream)))


def cache_gather(miss, n_miss, max_miss, host_store, slot_store, slab_bytes, stream=None):
    return _check("cache_gather", lib().cache_gather(_p(miss), _p(n_miss), max_miss, _p(host_store), _p(slot_store),
                                                     slab_bytes, _stream(stream)))


def moe_ffn_workspace_bytes(T, k, S, w_type, H, I) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, k, S, w_type, H, I))


def moe_ffn_slots(x, x_dtype, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y, ws, ws_bytes,
                  stream=None):
    return _check("moe_ffn_slots", lib().moe_ffn_slots(_p(x), x_dtype, _p(slot_ids), _p(w), T, k, _p(slot_store),
                                                       slab_bytes, S, w_type, H, I, _p(y), _p(ws), ws_bytes,
                                                       _stream(stream)))


def moe_ffn_slots_noalloc(x, x_dtype, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y, stream=None):
    return _check("moe_ffn_slots_noalloc",
                  lib().moe_ffn_slots_noalloc(_p(x), x_dtype, _p(slot_ids), _p(w), T, k, _p(slot_store), slab_bytes, S,
                                              w_type, H, I, _p(y), _stream(stream)))


def moe_ffn_noalloc_scratch_bytes() -> int:
    return int(lib().moe_ffn_noalloc_scratch_bytes())


def moe_ffn_host_misses(x_h, x_dtype, ids_h, slot_ids_h, w_h, T, k, host_store, slab_bytes, E, w_type, H, I, y_h,
                        n_threads):
    return _check("moe_ffn_host_misses", lib().moe_ffn_host_misses(_p(x_h), x_dtype, _p(ids_h), _p(slot_ids_h),
                                                                   _p(w_h), T, k, _p(host_store), slab_bytes, E,
                                                                   w_type, H, I, _p(y_h), n_threads))


def moe_combine(y, y_add, T, H, stream=None):
    return _check("moe_combine", lib().moe_combine(_p(y), _p(y_add), T, H, _stream(stream)))


def moe_residual(x, x_dtype, y, x_out, T, H, stream=None):
    return _check("moe_residual", lib().moe_residual(_p(x), x_dtype, _p(y), _p(x_out), T, H, _stream(stream)))


def moe_step_create(T_max, E, k, H, I, S, w_type):
    """Handle of the native step driver (owns its device / pinned buffers and events)."""
    h = lib().moe_step_create(T_max, E, k, H, I, S, w_type)
    if not h:
        raise MoeError("moe_step_create", MOE_E_NOMEM, (lib().moe_last_error() or b"").decode())
    return h


def moe_step_destroy(h):
    lib().moe_step_destroy(h)


def moe_step_output(h):
    return lib().moe_step_output(h)


def moe_step_stats(h, reset=False):
    out = (ctypes.c_int64 * 4)()
    _check("moe_step_stats", lib().moe_step_stats(h, out, int(reset)))
    return [int(v) for v in out]


def moe_layer_step(h, desc, x, T, ids_in, host_pass, n_threads, y_out, s0, s_side, s_copy):
    return _check("moe_layer_step", lib().moe_layer_step(h, ctypes.byref(desc), _p(x), T, _p(ids_in),
                                                         int(host_pass), n_threads, _p(y_out), _stream(s0),
                                                         _stream(s_side), _stream(s_copy)))


def moe_stack_step(h, descs, x, T, host_pass, n_threads, x_out, s0, s_side, s_copy):
    return _check("moe_stack_step", lib().moe_stack_step(h, descs, len(descs), _p(x), T, int(host_pass), n_threads,
                                                         _p(x_out), _stream(s0), _stream(s_side), _stream(s_copy)))


def moe_step_set_stream_threshold(h, picks_per_expert: int):
    return _check("moe_step_set_stream_threshold", lib().moe_step_set_stream_threshold(h, int(picks_per_expert)))


def moe_step_last_host_mode(h) -> int:
    return int(lib().moe_step_last_host_mode(h))


def moe_fused_spin_limit(polls: int = -1) -> int:
    """Polls of cache_manage_gather's copying workgroups before they give up;
    polls >= 0 sets it, < 0 queries.  Returns the previous limit."""
    return int(lib().moe_fused_spin_limit(int(polls)))


def moe_host_alloc(nbytes: int) -> int:
    p = lib().moe_host_alloc(nbytes)
    if not p:
        raise MoeError("moe_host_alloc", MOE_E_NOMEM, moe_last_error())
    return p


def moe_host_free(p: int):
    return _check("moe_host_free", lib().moe_host_free(p))

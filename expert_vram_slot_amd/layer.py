"""Call order of one expert-slot MoE layer step over the C ABI.

Holds the device and pinned-host buffers of one layer and issues the entry
points in the order the method needs them; it computes nothing itself.

Order of a step (sozai.app transcript "rtx-3060-run-35b-llamacpp": all GPU
work in one unbroken run, all CPU work in another, one add at the end;
"Porting vllm-expert-cache to NVIDIA GPUs": manage, gather, remap, expert
FFN over slot space):

  compute stream  moe_route -> cache_manage -> moe_ffn_slots ........ -> moe_combine
  side stream                    `-> cache_gather --^ (event)              ^
  copy stream     x -> host          `-> ids|slot_ids|w -> host (event)    |
  CPU thread                                  `-> moe_ffn_host_misses -> y_host

The GPU work is queued first and back to back (the CPU runs ahead of it), so
the device never waits for the host between the router and the FFN; the
host pass's inputs leave in two copies (x, and one packed block holding the
picks, their slots and their weights).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import torch

from . import (MOE_W_F32, MOE_X_BF16, MOE_X_F32, POLICIES, LayerDesc, cache_gather, cache_init, cache_manage,
               cache_state, moe_combine, moe_ffn_host_misses, moe_ffn_slots, moe_ffn_workspace_bytes, moe_layer_step,
               moe_residual, moe_route_ex, moe_slab_layout, moe_stack_step, moe_step_create,
               moe_step_destroy, moe_step_last_host_mode, moe_step_set_stream_threshold, moe_step_stats)


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class SlotLayer:
    def __init__(self, *, E, k, H, I, S, w_type, T_max, policy, host_store, slot_store, G, bias=None,
                 n_threads=None, device="cuda"):
        dev = torch.device(device)
        self.E, self.k, self.H, self.I, self.S = E, k, H, I, S
        self.w_type = w_type
        self.x_dtype = MOE_X_F32 if w_type == MOE_W_F32 else MOE_X_BF16
        self.policy = POLICIES.get(policy, policy)
        self.T_max = T_max
        self.slab = int(host_store.shape[1])
        assert moe_slab_layout(w_type, H, I).total <= self.slab
        self.host_store = host_store      # pinned [E][slab] uint8
        self.slot_store = slot_store      # device [S][slab] uint8
        self.G, self.bias = G, bias
        self.n_threads = n_threads or host_threads()
        P = T_max * k
        self.P_max = P
        i32 = dict(dtype=torch.int32, device=dev)
        # picks, their slots and their weights in one block (one copy to the host)
        self.meta = torch.empty(3 * P, **i32)
        self.ids = self.meta[:P]
        self.slot_ids = self.meta[P:2 * P]
        self.w = self.meta[2 * P:].view(torch.float32)
        # router logits (also lets the router run as logits + top-k kernels)
        self.logits = torch.empty(T_max * E, dtype=torch.float32, device=dev)
        self.miss = torch.empty(2 * max(S, 1), **i32)
        self.n_miss = torch.zeros(1, **i32)
        self.host_miss = torch.empty(E, **i32)
        self.n_host = torch.zeros(1, **i32)
        self.stats = torch.zeros(4, **i32)
        self.e2s = torch.empty(E, **i32)
        self.s2e = torch.empty(max(S, 1), **i32)
        self.last = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
        self.freq = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
        self.step_ctr = torch.zeros(1, dtype=torch.int32, device=dev)
        self.st = cache_state(self.e2s, self.s2e, self.last, self.freq, self.step_ctr, E, S)
        self.ws_bytes = moe_ffn_workspace_bytes(T_max, k, max(S, 1), w_type, H, I)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.y = torch.empty(T_max * H, dtype=torch.float32, device=dev)
        self.y_host_dev = torch.empty(T_max * H, dtype=torch.float32, device=dev)
        xb = 4 if self.x_dtype == MOE_X_F32 else 2
        pin = dict(pin_memory=True)
        self.h_x = torch.empty(T_max * H * xb, dtype=torch.uint8, **pin)
        self.h_meta = torch.empty(3 * P, dtype=torch.int32, **pin)
        self.h_ids = self.h_meta[:P]
        self.h_slot = self.h_meta[P:2 * P]
        self.h_w = self.h_meta[2 * P:].view(torch.float32)
        self.h_y = torch.empty(T_max * H, dtype=torch.float32, **pin)
        self.side = torch.cuda.Stream(device=dev)
        self.copy = torch.cuda.Stream(device=dev)
        self.pool = cf.ThreadPoolExecutor(max_workers=1)
        self.ffn_events = None     # (start, end) torch events recorded around moe_ffn_slots when set
        self.gather_events = None  # (start, end) torch events recorded around cache_gather when set
        self.route_flags = 0       # moe_route_ex flags (MOE_ROUTE_DAMPED)

    def init_cache(self, resident=None):
        cache_init(self.st, resident)

    def _host_pass(self, ev, T):
        ev.synchronize()
        moe_ffn_host_misses(self.h_x, self.x_dtype, self.h_ids, self.h_slot, self.h_w, T, self.k, self.host_store,
                            self.slab, self.E, self.w_type, self.H, self.I, self.h_y, self.n_threads)

    def step(self, x, T, ids_in=None, host_pass=True):
        """One layer step for T tokens of x (device, [T][H]); returns y [T][H] fp32 (device)."""
        assert T <= self.T_max
        cur = torch.cuda.current_stream()
        P = T * self.k
        if host_pass:
            # 0. the host pass's activations leave while the router runs
            self.copy.wait_stream(cur)
            with torch.cuda.stream(self.copy):
                nx = x.numel() * x.element_size()
                self.h_x[:nx].copy_(x.reshape(-1).view(torch.uint8), non_blocking=True)
        if ids_in is not None:
            # given picks are copied into the packed block (the host pass reads them from there)
            self.ids[:P].copy_(ids_in.reshape(-1)[:P], non_blocking=True)
        # 1. router (picks, or weights of given picks)
        moe_route_ex(x, self.x_dtype, self.G, self.bias, None if ids_in is None else self.ids, T, self.H, self.E,
                     self.k, self.route_flags, self.ids, self.w, self.logits, cur)
        ids = self.ids
        # 2. cache step: victims, miss list, remap
        cache_manage(self.st, self.policy, ids, P, self.slot_ids, self.miss, self.n_miss, self.host_miss,
                     self.n_host, self.stats, cur)
        ev_manage = torch.cuda.Event()
        ev_manage.record(cur)
        # 3. gather on the side stream (a static cache never loads while running)
        if self.policy != 0 and self.S > 0:
            self.side.wait_event(ev_manage)
            gev = self.gather_events
            if gev:
                gev[0].record(self.side)
            cache_gather(self.miss, self.n_miss, self.S, self.host_store, self.slot_store, self.slab, self.side)
            if gev:
                gev[1].record(self.side)
            ev_g = torch.cuda.Event()
            ev_g.record(self.side)
            cur.wait_event(ev_g)
        # 4. expert FFN over resident slots (zero for the rest); optional timing events around it
        ev = getattr(self, "ffn_events", None)
        if ev:
            ev[0].record(cur)
        moe_ffn_slots(x, self.x_dtype, self.slot_ids, self.w, T, self.k, self.slot_store, self.slab, max(self.S, 1),
                      self.w_type, self.H, self.I, self.y, self.ws, self.ws_bytes, cur)
        if ev:
            ev[1].record(cur)
        if host_pass:
            # 5. picks, slots and weights to pinned memory (one copy), then the host pass on CPU threads
            self.copy.wait_event(ev_manage)
            with torch.cuda.stream(self.copy):
                self.h_meta.copy_(self.meta, non_blocking=True)
                ev_copy = torch.cuda.Event()
                ev_copy.record(self.copy)
            fut = self.pool.submit(self._host_pass, ev_copy, T)
            # 6. the single add joining the two passes
            fut.result()
            self.y_host_dev[:T * self.H].copy_(self.h_y[:T * self.H], non_blocking=True)
            moe_combine(self.y, self.y_host_dev, T, self.H, cur)
        return self.y[:T * self.H].view(T, self.H)


class SlotStack:
    """Stacked expert-slot MoE layers joined by a residual stream kept in the
    activation format: x_{l+1} = x_l + y_l ("Nudge, don't cut", "Experts that
    don't fit": a deep model of routed layers).

    Each layer brings its pinned host store, slot store, router gate,
    optional bias table and static resident set; the step buffers, streams
    and host-pass worker are shared by all layers (they run one after the
    other).
    """

    def __init__(self, *, E, k, H, I, S, w_type, T_max, layers, n_threads=None, device="cuda"):
        self.layers = layers
        first = layers[0]
        self.layer = SlotLayer(E=E, k=k, H=H, I=I, S=S, w_type=w_type, T_max=T_max, policy="static",
                               host_store=first["host_store"], slot_store=first["slot_store"], G=first["G"],
                               bias=first.get("bias"), n_threads=n_threads, device=device)
        dev = torch.device(device)
        self.states = []
        for spec in layers:
            e2s = torch.empty(E, dtype=torch.int32, device=dev)
            s2e = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
            last = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
            freq = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
            step = torch.zeros(1, dtype=torch.int32, device=dev)
            st = cache_state(e2s, s2e, last, freq, step, E, S)
            cache_init(st, spec["resident"])
            self.states.append((st, e2s, s2e, last, freq, step))
        xb = 4 if self.layer.x_dtype == MOE_X_F32 else 2
        self.xbuf = [torch.empty(T_max * H * xb, dtype=torch.uint8, device=dev) for _ in range(2)]
        self.H = H

    def bind(self, l):
        """Point the shared step machinery at layer l."""
        L, spec = self.layer, self.layers[l]
        L.host_store, L.slot_store, L.G, L.bias = spec["host_store"], spec["slot_store"], spec["G"], spec.get("bias")
        L.st = self.states[l][0]
        return L

    def step(self, x, T, host_pass=True, trace=None, on_layer=None, ffn_events=None):
        """All layers for T tokens of x (device [T][H] in the activation
        format); returns the last layer's residual output (a view of an
        internal buffer).  `trace`, if a list, receives per layer a copy of
        (x_l, ids, slot_ids, w, y_l) for checking; `on_layer(l, L, x_l, y_l)`
        is called after each layer's step; `ffn_events`, if a list, receives
        per layer the (start, end) events around moe_ffn_slots."""
        cur = x.reshape(-1)
        nb = T * self.H * (4 if self.layer.x_dtype == MOE_X_F32 else 2)
        for l in range(len(self.layers)):
            L = self.bind(l)
            if ffn_events is not None:
                L.ffn_events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ffn_events.append(L.ffn_events)
            xl = cur.view(x.dtype).view(T, self.H)
            y = L.step(xl, T, host_pass=host_pass)
            L.ffn_events = None
            if trace is not None:
                P = T * L.k
                trace.append((xl.clone(), L.ids[:P].clone(), L.slot_ids[:P].clone(), L.w[:P].clone(), y.clone()))
            if on_layer is not None:
                on_layer(l, L, xl, y)
            nxt = self.xbuf[l % 2][:nb]
            moe_residual(cur, L.x_dtype, y, nxt, T, self.H)
            cur = nxt
        return cur.view(x.dtype).view(T, self.H)


class NativeStack:
    """The same layers as SlotStack driven by the library's native step
    driver (moe_layer_step / moe_stack_step): one call per layer or per whole
    stack, no Python between the entry points of a step.

    layers: list of dicts with host_store (pinned), slot_store, G, bias (or
    None), resident (device int32 [S], or None for an empty dynamic cache)
    and optionally policy ("static" by default).
    """

    def __init__(self, *, E, k, H, I, S, w_type, T_max, layers, n_threads=None, device="cuda"):
        dev = torch.device(device)
        self.E, self.k, self.H, self.I, self.S, self.T_max = E, k, H, I, S, T_max
        self.x_dtype = MOE_X_F32 if w_type == MOE_W_F32 else MOE_X_BF16
        self.n_threads = n_threads or host_threads()
        self.h = moe_step_create(T_max, E, k, H, I, S, w_type)
        self.side = torch.cuda.Stream(device=dev)
        self.copy = torch.cuda.Stream(device=dev)
        self.keep = []  # tensors the descriptors point at
        descs = (LayerDesc * len(layers))()
        for i, spec in enumerate(layers):
            i32 = dict(dtype=torch.int32, device=dev)
            st_t = [torch.empty(E, **i32), torch.empty(max(S, 1), **i32), torch.empty(max(S, 1), **i32),
                    torch.empty(max(S, 1), **i32), torch.zeros(1, **i32)]
            st = cache_state(*st_t, E, S)
            cache_init(st, spec.get("resident"))
            self.keep.append((st_t, spec))
            d = descs[i]
            d.G = spec["G"].data_ptr()
            d.bias = spec["bias"].data_ptr() if spec.get("bias") is not None else None
            d.state = st
            d.policy = POLICIES.get(spec.get("policy", "static"), spec.get("policy", 0))
            d.slot_store = spec["slot_store"].data_ptr()
            d.host_store = spec["host_store"].data_ptr()
            d.slab_bytes = int(spec["host_store"].shape[1])
        self.descs = descs
        xb = 4 if self.x_dtype == MOE_X_F32 else 2
        self.out = torch.empty(T_max * H * xb, dtype=torch.uint8, device=dev)
        self.y = torch.empty(T_max * H, dtype=torch.float32, device=dev)

    def e2s(self, l):
        return self.keep[l][0][0]

    def init_cache(self, l, resident=None):
        """Set layer l's cache state again (resident: device int32 [S], or None: empty)."""
        cache_init(self.descs[l].state, resident)

    def layer_step(self, l, x, T, ids_in=None, host_pass=True):
        """One layer; returns y [T][H] fp32 (a view of this object's output buffer)."""
        moe_layer_step(self.h, self.descs[l], x, T, ids_in, host_pass, self.n_threads, self.y,
                       torch.cuda.current_stream(), self.side, self.copy)
        return self.y[:T * self.H].view(T, self.H)

    def step(self, x, T, host_pass=True):
        """All layers with the residual join; returns the last residual output [T][H]."""
        moe_stack_step(self.h, self.descs, x, T, host_pass, self.n_threads, self.out, torch.cuda.current_stream(),
                       self.side, self.copy)
        nb = T * self.H * (4 if self.x_dtype == MOE_X_F32 else 2)
        return self.out[:nb].view(x.dtype).view(T, self.H)

    def stats(self, reset=False):
        return moe_step_stats(self.h, reset)

    def set_stream_threshold(self, picks_per_expert):
        """Picks per non-resident expert from which a step streams its misses (0: always, < 0: never)."""
        moe_step_set_stream_threshold(self.h, picks_per_expert)

    def last_host_mode(self):
        """0: no host misses, 1: the CPU lane, 2: streamed through the GPU (last layer step)."""
        return moe_step_last_host_mode(self.h)

    def close(self):
        if self.h:
            moe_step_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


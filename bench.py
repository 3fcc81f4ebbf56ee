"""Benchmark of the expert-slot MoE layer on one MI355X.

Workload: one Qwen3-30B-A3B-shaped MoE layer in bf16 (128 experts, top-8,
hidden 2048, expert intermediate 768, SwiGLU), decode batch of 64 tokens, a
static 64-slot VRAM cache chosen from a 1,024-token profile batch; the other
64 experts sit in pinned host memory and are served by the CPU host pass.
Synthetic, seeded inputs: weights ~N(0, 0.02), router gate ~N(0, 0.05),
activations ~N(0, 1) fresh per step.

A step is one pass of the whole path over one batch: moe_route ->
cache_manage -> cache_gather (side stream; nothing to copy under a static
cache) -> moe_ffn_slots on the GPU, concurrently moe_ffn_host_misses on CPU
threads -> moe_combine.  Inputs are resident in HBM when the timed region
starts.  Four layer copies with distinct weights rotate so that the 256 MB
Infinity Cache cannot hold the expert weights between steps.

Printed: one JSON line (metric of the layer: tokens/s), with the slot FFN's
expert-weight HBM rate against the 8 TB/s peak (HIP events around every
moe_ffn_slots launch of the timed steps), the gather rate against the
measured host link, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64, help="decode tokens per step (1, 8 or 64)")
    ap.add_argument("--layers", type=int, default=4, help="distinct layer copies rotated per step")
    ap.add_argument("--threads", type=int, default=0, help="host-pass threads (0: min(16, cores))")
    ap.add_argument("--no-host-pass", action="store_true", help="GPU pass only (not the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes, for scaling HBM counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the expert-slot layer is a single-GPU path here "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 1 << 30, "launches": args.steps}))
        return

    import expert_vram_slot_amd as m
    import synth
    from expert_vram_slot_amd.layer import SlotLayer, host_threads

    cfg = "c2"
    c = synth.CONFIGS[cfg]
    E, k, H, I, S = c["E"], c["k"], c["H"], c["I"], c["S"]
    T = args.batch
    w_type, x_dtype = c["w_type"], c["x_dtype"]
    base = synth.config_seed(cfg)
    slab = synth.slab_bytes(w_type, H, I)
    nthreads = args.threads or host_threads()
    dev = torch.device("cuda")
    torch.cuda.set_device(0)

    # ---- per-layer inputs: pinned host store, router gate, static resident set, slot store
    layers = []
    n_x = 8
    for l in range(args.layers):
        store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
        synth.slabs_into(store.data_ptr(), w_type, base, l, 0, E, H, I, c["sigma_w"], slab)
        G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, l), (E, H), c["sigma_g"], x_dtype)
                             .view(np.int16)).to(dev)
        # profile batch (different seed tag) -> the S most-picked experts, on the GPU
        warm = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_WARM, l), (1024, H), 1.0, x_dtype)
                                .view(np.int16)).to(dev)
        wids = torch.empty((1024, k), dtype=torch.int32, device=dev)
        ww = torch.empty((1024, k), dtype=torch.float32, device=dev)
        m.moe_route(warm, x_dtype, G, None, None, 1024, H, E, k, wids, ww, None)
        resident = torch.empty(S, dtype=torch.int32, device=dev)
        m.cache_pick_static(wids, 1024 * k, E, S, resident)
        torch.cuda.synchronize()
        res_h = resident.cpu().numpy()
        slots = store[torch.from_numpy(res_h.astype(np.int64))].to(dev)
        L = SlotLayer(E=E, k=k, H=H, I=I, S=S, w_type=w_type, T_max=T, policy="static", host_store=store,
                      slot_store=slots, G=G, n_threads=nthreads)
        L.init_cache(resident)
        xs = [torch.from_numpy(synth.normal(synth.key(base, synth.TAG_X, l, s), (T, H), 1.0, x_dtype)
                               .view(np.int16)).to(dev) for s in range(n_x)]
        layers.append((L, xs))
    torch.cuda.synchronize()

    # ---- timed steps; events around every moe_ffn_slots launch (compute stream)
    ffn_ms = []
    ffn_bytes = []
    ev_pairs = []

    def one_step(i, record):
        L, xs = layers[i % len(layers)]
        x = xs[(i // len(layers)) % n_x]
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            L.ffn_events = (e0, e1)
        else:
            L.ffn_events = None
        L.step(x, T, host_pass=not args.no_host_pass)
        if record:
            ev_pairs.append((e0, e1, L))

    for i in range(args.warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for e0, e1, L in ev_pairs:
        ffn_ms.append(e0.elapsed_time(e1))
    ms_per_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed

    # algorithmic bytes of one moe_ffn_slots launch: every distinct resident slab the step touched, read
    # once, plus x in and y out.  Distinct slabs per step: rerun each timed step's routing (untimed).
    distinct = []
    for i in range(args.steps):
        L, xs = layers[(args.warmup + i) % len(layers)]
        x = xs[((args.warmup + i) // len(layers)) % n_x]
        m.moe_route(x, x_dtype, L.G, None, None, T, H, E, k, L.ids, L.w, None)
        torch.cuda.synchronize()
        ids = L.ids[:T * k].cpu().numpy()
        e2s = L.e2s.cpu().numpy()
        sl = e2s[ids]
        distinct.append(len(set(sl[sl >= 0].tolist())))
    act_bytes = T * H * 2 + T * H * 4  # x (bf16) in, y (fp32) out
    per_launch = [d * slab + act_bytes for d in distinct]
    ffn_ms_arr = np.array(ffn_ms)
    achieved = float(np.mean(per_launch) / (np.mean(ffn_ms_arr) * 1e-3) / 1e9)

    out = {
        "metric": "MoE-layer tokens/s; expert-weight HBM GB/s as % of peak; gather GB/s",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"qwen3-30b-a3b-shaped MoE layer, bf16, E=128 top-8, H=2048 I=768, decode T={T}, "
                               f"static 64-slot cache + host pass of the other 64 experts",
                   "global_batch": T, "layers_rotated": args.layers, "host_threads": nthreads,
                   "host_pass": not args.no_host_pass},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "moe_ffn_slots (group, gate/up, down, reduce kernels)",
                     "bytes_per_launch": int(np.mean(per_launch)), "ms_per_launch": round(float(np.mean(ffn_ms_arr)), 5),
                     "distinct_slabs_per_step": round(float(np.mean(distinct)), 2)},
    }

    if not args.no_gather:
        out["gather"] = measure_gather(m, torch, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth, T)
    print(json.dumps(out), flush=True)


def measure_gather(m, torch, synth):
    """cache_gather of whole W8A8 expert slabs (4,732,928 B) from pinned host
    memory into slots, against a plain pinned hipMemcpyAsync of the same bytes."""
    E, S = 128, 32
    slab = synth.slab_bytes(synth.W_W8A8, 2048, 768)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    store.view(-1)[::4096].fill_(7)
    slots = torch.empty((S, slab), dtype=torch.uint8, device="cuda")
    n = S
    miss = torch.tensor(np.stack([np.arange(n) * 3 % E, np.arange(n)], 1).reshape(-1), dtype=torch.int32,
                        device="cuda")
    n_miss = torch.tensor([n], dtype=torch.int32, device="cuda")
    for _ in range(2):
        m.cache_gather(miss, n_miss, S, store, slots, slab)
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        m.cache_gather(miss, n_miss, S, store, slots, slab)
    e1.record()
    torch.cuda.synchronize()
    g_gbs = reps * n * slab / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # host link: pinned H2D copy engine, same bytes
    src = store[:n].reshape(-1)
    dst = slots.reshape(-1)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    link = reps * n * slab / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"gbs": round(g_gbs, 2), "link_gbs": round(link, 2), "frac": round(g_gbs / link, 4),
            "slab_bytes": slab, "slabs_per_call": n, "link": "pinned hipMemcpyAsync H2D"}


def cpu_baseline(synth, T):
    """The oracle (single-threaded C) on a bounded sample of the same workload:
    logits, top-k, weights and the full SwiGLU layer for 8 tokens."""
    import oracle
    li = synth.LayerInputs("c2", T=8)
    t0 = time.perf_counter()
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, li.k)
    w = oracle.route_weights(z, ids)
    oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids, w)
    dt = time.perf_counter() - t0
    return {"value": round(8 / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "8 tokens of the same layer (route + full SwiGLU layer in double), single thread"}


if __name__ == "__main__":
    main()

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
measured host link, and the CPU oracle's rate on a bounded sample.  The same
line carries two more workloads of the layer:

  prefill  the 288-expert bf16 layer (hidden 4096, intermediate 1536, top-8)
           on 2048 tokens, every expert resident (10.9 GB of slots): route ->
           manage -> moe_ffn_slots on the MFMA grouped GEMM; HBM and MFMA
           fractions; plus the same layer at 16384 tokens, the shape where
           the grouped GEMM is compute-bound (supplemental)
  decode_batches  the same bf16 layer's FFN at 1, 8 and 64 tokens per step:
           expert-weight GB/s against the HBM peak
  prefill_144  the 288-expert layer at 2048 tokens with 144 experts resident
           and 144 in pinned host memory, served by the step as the native
           driver chooses (streamed through staging slots at this batch), and
           with the CPU lane forced
  dynamic  the 128-expert W8A8 layer under Zipf(0.8) routing with a 32-slot
           LRU cache, 256 steps of 16 tokens from an empty cache: hit rate per
           routing id, experts gathered per step, gather GB/s against the
           measured host link, layer tokens/s with the host pass
  stack    the 48-layer, 512-expert top-10 4-bit stack (43.5 GB pinned host
           store, 192 resident experts per layer, graded bias cap -1) at 1
           and 32 tokens: tokens/s, the FFN's expert-weight GB/s, hit rates
           with and without the bias (--no-stack leaves it out)

`--workload stack` runs only the 48-layer, 512-expert 4-bit stack,
`--workload bias` the routing-bias variants (flat bias, hard mask, graded
table, damped weights; live-cache affinity on a dynamic cache), and
`--workload replay` a routing trace replayed under the cache policies
(static, LRU, LFU, periodic repick, the perfect-foresight fixed set).
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
MFMA_BF16_PEAK_TFS = 2500.0

# kernels launched, in order, by one moe_ffn_slots call on the bf16 decode layer: at 64 tokens (512 picks) the
# MFMA gate/up GEMM on decode-shaped tiles (which sorts the picks itself), the down GEMM and the reduction; at 1
# and 8 tokens the pick sort and the row-streaming gate/up and down kernels, then the reduction.  The first
# name anchors a launch; the names before it are the closest earlier dispatches, those after it the closest
# later ones.
FFN_SEQS = {64: ((), "k_dec_gemm<0, 4, 2, false>", ("k_dec_gemm<1, 4, 2, false>", "k_reduce")),
            8: (("k_group_small",), "k_gu<1, 4, false>", ("k_down<1, 3, 32>", "k_reduce")),
            1: ((), "k_gu<1, 4, true>", ("k_down_tok<1, 3, 32>",))}
# source files whose change invalidates stored HBM counter readings of those kernels
FFN_SOURCES = ("expert_vram_slot_amd/csrc/ffn.hip", "expert_vram_slot_amd/csrc/prefill.hip",
               "expert_vram_slot_amd/csrc/prefill.hpp", "expert_vram_slot_amd/csrc/common.hpp")
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--replicate", type=int, default=0,
                    help="run the benchmark this many times in fresh processes and print one line with the median "
                         "value and the min-max of the headline figures")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64, help="decode tokens per step (1, 8 or 64)")
    ap.add_argument("--layers", type=int, default=4, help="distinct layer copies rotated per step")
    ap.add_argument("--threads", type=int, default=0, help="host-pass threads (0: min(16, cores))")
    ap.add_argument("--no-host-pass", action="store_true", help="GPU pass only (not the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-dynamic", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="leave out the 48-layer 4-bit stack leg")
    ap.add_argument("--no-extra-batches", action="store_true",
                    help="time only --batch on the decode layer (not also 1 and 8 tokens)")
    ap.add_argument("--summarize-kernels", nargs=5, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                             "COPY_WRITE_DIR"), default=None,
                    help="write a per-kernel summary (time, scaled HBM counters) of any profiled run to --out, "
                         "titled --title")
    ap.add_argument("--title", default="")
    ap.add_argument("--workload", choices=["decode", "stack", "bias", "replay"], default="decode")
    ap.add_argument("--stack-steps", type=int, default=20, help="timed 48-layer steps at T=1 (half at T=32)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes, for scaling HBM counters)")
    ap.add_argument("--summarize", nargs=5, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                     "COPY_WRITE_DIR"),
                    help="write a text summary of rocprofv3 CSV output (kernel trace + FETCH_SIZE/WRITE_SIZE runs of "
                         "this benchmark and of --copy-calibration) to --out; no GPU needed")
    ap.add_argument("--summarize-prefill", nargs=5, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                              "COPY_WRITE_DIR"), default=None,
                    help="write the prefill kernels' summary (2048- and 16384-token legs) from the same runs")
    ap.add_argument("--prefill-mfma", default=None, metavar="MFMA_DIR",
                    help="with --summarize-prefill: a run of this benchmark with --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                         "GRBM_GUI_ACTIVE MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16, summarised per prefill kernel")
    ap.add_argument("--out", default=None, help="summary file for --summarize")
    ap.add_argument("--commands", default=None, help="text file with the profiling commands, quoted in the summary")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.summarize_prefill:
        summarize_prefill(args)
        return
    if args.summarize_kernels:
        summarize_kernels(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the expert-slot layer is a single-GPU path here "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    if args.replicate > 0:
        replicate(args.replicate)
        return

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
    from expert_vram_slot_amd.layer import NativeStack, SlotLayer, SlotStack, host_threads

    if args.workload == "stack":
        out = bench_stack(m, torch, synth, SlotStack, NativeStack, args.threads or host_threads(), args)
        print(json.dumps(out), flush=True)
        return
    if args.workload == "bias":
        out = bench_bias(m, torch, synth, SlotLayer, NativeStack, args.threads or host_threads())
        print(json.dumps(out), flush=True)
        return
    if args.workload == "replay":
        print(json.dumps(bench_replay(m, torch, synth)), flush=True)
        return

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
    specs = []
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
        specs.append(dict(host_store=store, slot_store=slots, G=G, bias=None, resident=resident))
    # the layer step as a user runs it: the library's native driver, one call per step
    native = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=w_type, T_max=T, layers=specs, n_threads=nthreads)
    torch.cuda.synchronize()

    def native_step(i):
        l = i % len(layers)
        native.layer_step(l, layers[l][1][(i // len(layers)) % n_x], T, host_pass=not args.no_host_pass)

    for i in range(args.warmup):
        native_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        native_step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed

    # ---- the same steps again on the GPU alone (route -> manage -> moe_ffn_slots, no host pass), issued
    # from Python with HIP events around every moe_ffn_slots launch on the compute stream: the FFN's
    # duration for the roofline, free of gaps from CPU threads competing with the launching thread
    t1 = time.perf_counter()
    ffn_ms_arr, per_launch, distinct, b2b_ms = gpu_ffn_pass(m, torch, layers, n_x, T, args.steps, args.warmup,
                                                            x_dtype, H, E, k, slab)
    elapsed_py = time.perf_counter() - t1
    achieved = float(np.mean(per_launch) / (np.mean(ffn_ms_arr) * 1e-3) / 1e9)
    # the smaller decode batches of the same layer (same layers, same steps, first T rows of x)
    batches = {}
    for Tb in (() if args.no_extra_batches else (1, 8)):
        ms_b, pl_b, d_b, b2b_b = gpu_ffn_pass(m, torch, layers, n_x, Tb, args.steps, args.warmup, x_dtype, H, E, k,
                                              slab)
        gbs = float(np.mean(pl_b) / (np.mean(ms_b) * 1e-3) / 1e9)
        gbs_b2b = float(np.mean(pl_b) / (b2b_b * 1e-3) / 1e9)
        batches[f"T{Tb}"] = {"ffn_us": round(float(np.mean(ms_b)) * 1e3, 2), "bytes_per_launch": int(np.mean(pl_b)),
                             "distinct_slabs_per_step": round(float(np.mean(d_b)), 2), "gbs": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "ffn_us_back_to_back": round(b2b_b * 1e3, 2),
                             "hbm_frac_back_to_back": round(gbs_b2b / HBM_PEAK_GBS, 4)}
    gbs64_b2b = float(np.mean(per_launch) / (b2b_ms * 1e-3) / 1e9)
    batches["T64"] = {"ffn_us": round(float(np.mean(ffn_ms_arr)) * 1e3, 2), "bytes_per_launch": int(np.mean(per_launch)),
                      "distinct_slabs_per_step": round(float(np.mean(distinct)), 2), "gbs": round(achieved, 1),
                      "hbm_frac": round(achieved / HBM_PEAK_GBS, 4), "ffn_us_back_to_back": round(b2b_ms * 1e3, 2),
                      "hbm_frac_back_to_back": round(gbs64_b2b / HBM_PEAK_GBS, 4)}

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
                   "host_pass": not args.no_host_pass, "driver": "native moe_layer_step",
                   "gpu_only_step_ms": round(elapsed_py / args.steps * 1e3, 4),
                   "step_bound_by": ("the CPU host pass: the 64 non-resident experts' slabs (604 MB) are read from "
                                     "pinned host memory every step" if not args.no_host_pass else "the GPU")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(T),
                     "kernel": "moe_ffn_slots (pick sort, MFMA gate/up and down grouped GEMMs, reduction)",
                     "bytes_per_launch": int(np.mean(per_launch)), "ms_per_launch": round(float(np.mean(ffn_ms_arr)), 5),
                     "distinct_slabs_per_step": round(float(np.mean(distinct)), 2)},
        "decode_batches": dict(batches, workload="the same 128-expert bf16 layer, 64 resident slots, moe_ffn_slots "
                                                 "alone, 4 layer copies rotated; ffn_us: HIP events around each "
                                                 "launch; ffn_us_back_to_back: the same launches (each step's picks "
                                                 "and weights kept) issued back to back, one pair of events around "
                                                 "them all"),
    }

    del layers, specs
    native.close()
    del native
    release(torch)
    link = None
    if not args.no_gather:
        out["gather"] = measure_gather(m, torch, synth)
        link = out["gather"]["link_gbs"]
        release(torch)
    if not args.no_prefill:
        out["prefill"], store5 = bench_prefill(m, torch, synth, SlotLayer)
        out["prefill_144"] = bench_prefill_144(m, torch, synth, NativeStack, store5, nthreads)
        del store5
        release(torch)
    if not args.no_dynamic:
        out["dynamic"] = bench_dynamic(m, torch, synth, SlotLayer, NativeStack, nthreads, link)
        release(torch)
    if not args.no_stack:
        st = bench_stack(m, torch, synth, SlotStack, NativeStack, nthreads, args)
        out["stack"] = {key: st[key] for key in ("workload", "T1", "T32")}
        release(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth, T)
    print(json.dumps(out), flush=True)


def release(torch):
    """Hand the memory of finished legs back: device memory and pinned host
    memory that torch keeps cached (the 48-layer stack pins 43.5 GB)."""
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if hasattr(torch._C, "_host_emptyCache"):
        torch._C._host_emptyCache()


def gpu_ffn_pass(m, torch, layers, n_x, T, steps, warmup, x_dtype, H, E, k, slab):
    """route -> manage -> moe_ffn_slots for T tokens over the rotated layers,
    no host pass, HIP events around every moe_ffn_slots launch; returns the
    per-launch times (ms), the algorithmic bytes of each launch (every
    distinct resident slab the step touched, read once, plus x in and y out),
    the distinct slabs per step (from rerunning each step's routing, untimed)
    and the mean time per launch of the same launches issued back to back
    (each step's picks and weights kept, one pair of events around them all:
    no event packets between the launches)."""
    ev_pairs = []
    kept = []

    def one_step(i, record):
        L, xs = layers[i % len(layers)]
        x = xs[(i // len(layers)) % n_x][:T]
        if record:
            L.ffn_events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        else:
            L.ffn_events = None
        L.step(x, T, host_pass=False)
        if record:
            ev_pairs.append(L.ffn_events)
            kept.append((L, x, L.slot_ids[:T * k].clone(), L.w[:T * k].clone()))
        L.ffn_events = None

    for i in range(warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    for i in range(steps):
        one_step(warmup + i, True)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev_pairs])
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for L, x, sl, w in kept:
        m.moe_ffn_slots(x, x_dtype, sl, w, T, k, L.slot_store, L.slab, max(L.S, 1), L.w_type, H, L.I, L.y, L.ws,
                        L.ws_bytes, cur)
    e1.record(cur)
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / len(kept)
    distinct = []
    for i in range(steps):
        L, xs = layers[(warmup + i) % len(layers)]
        x = xs[((warmup + i) // len(layers)) % n_x][:T]
        m.moe_route(x, x_dtype, L.G, None, None, T, H, E, k, L.ids, L.w, None)
        torch.cuda.synchronize()
        ids = L.ids[:T * k].cpu().numpy()
        sl = L.e2s.cpu().numpy()[ids]
        distinct.append(len(set(sl[sl >= 0].tolist())))
    act_bytes = T * H * 2 + T * H * 4  # x (bf16) in, y (fp32) out
    return ms, [d * slab + act_bytes for d in distinct], distinct, b2b_ms


def bench_prefill(m, torch, synth, SlotLayer, steps=10, warmup=2):
    """The 288-expert prefill layer, all experts resident; one step = route ->
    manage -> moe_ffn_slots for 2048 tokens (no host pass: nothing misses)."""
    c = synth.CONFIGS["c5"]
    E, k, H, I, T = c["E"], c["k"], c["H"], c["I"], c["T"]
    base = synth.config_seed("c5")
    slab = synth.slab_bytes(synth.W_BF16, H, I)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)  # also the 144-slot variant's host store
    synth.slabs_into(store.data_ptr(), synth.W_BF16, base, 0, 0, E, H, I, c["sigma_w"], slab)
    slots = store.cuda()
    G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, 0), (E, H), c["sigma_g"], 1).view(np.int16)).cuda()
    xs = [torch.from_numpy(synth.normal(synth.key(base, synth.TAG_X, 0, st), (T, H), 1.0, 1).view(np.int16)).cuda()
          for st in range(2)]
    L = SlotLayer(E=E, k=k, H=H, I=I, S=E, w_type=synth.W_BF16, T_max=T, policy="static", host_store=store,
                  slot_store=slots, G=G)
    L.init_cache(torch.arange(E, dtype=torch.int32, device="cuda"))
    ev = []
    for i in range(warmup + steps):
        rec = i >= warmup
        if i == warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        L.ffn_events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if rec else None
        L.step(xs[i % 2], T, host_pass=False)
        if rec:
            ev.append(L.ffn_events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    P = T * k
    byts = E * slab + T * H * 2 + T * H * 4  # every slab is touched at 2048 tokens
    flops = 2.0 * P * 3 * H * I
    out = {"workload": "288-expert bf16 MoE layer, H=4096 I=1536 top-8, 2048 tokens, all 288 experts resident",
           "tokens_per_s": round(T * steps / elapsed, 1), "ms_per_step": round(elapsed / steps * 1e3, 4),
           "ffn_ms": round(ffn_ms, 4), "ffn_gbs": round(byts / ffn_ms / 1e6, 1),
           "hbm_frac": round(byts / ffn_ms / 1e6 / HBM_PEAK_GBS, 4),
           "ffn_tflops": round(flops / ffn_ms / 1e9, 1),
           "mfma_frac": round(flops / ffn_ms / 1e9 / MFMA_BF16_PEAK_TFS, 4)}
    # supplemental: 16384 tokens (about 455 rows per expert), where the grouped GEMM is compute-bound
    T2 = 16384
    x2 = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_X, 0, 99), (T2, H), 1.0, 1).view(np.int16)).cuda()
    ids = torch.empty((T2, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T2, k), dtype=torch.float32, device="cuda")
    m.moe_route(x2, 1, G, None, None, T2, H, E, k, ids, w, None)
    ws_b = m.moe_ffn_workspace_bytes(T2, k, E, 1, H, I)
    ws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    y = torch.empty((T2, H), dtype=torch.float32, device="cuda")
    for _ in range(3):  # warm-up, as for the 2048-token steps
        m.moe_ffn_slots(x2, 1, ids, w, T2, k, slots, slab, E, 1, H, I, y, ws, ws_b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n2 = 5
    e0.record()
    for _ in range(n2):
        m.moe_ffn_slots(x2, 1, ids, w, T2, k, slots, slab, E, 1, H, I, y, ws, ws_b)
    e1.record()
    torch.cuda.synchronize()
    ms2 = e0.elapsed_time(e1) / n2
    flops2 = 2.0 * T2 * k * 3 * H * I
    out["supplemental_16384_tokens"] = {"ffn_ms": round(ms2, 3), "ffn_tflops": round(flops2 / ms2 / 1e9, 1),
                                        "mfma_frac": round(flops2 / ms2 / 1e9 / MFMA_BF16_PEAK_TFS, 4)}
    del L, slots, ws, x2, y
    return out, store


def bench_prefill_144(m, torch, synth, NativeStack, store, nthreads, steps=3):
    """The 144-slot variant of the 288-expert layer at 2048 tokens: the 144
    most-picked experts of a 1024-token profile batch resident, the other 144
    in pinned host memory, served by the step itself.  Timed with the native
    driver as it chooses (at this batch: streamed through the GPU's staging
    slots), then with the CPU lane forced, and on the GPU alone (the
    non-resident picks add zero) for the CPU lane's overlap."""
    c = synth.CONFIGS["c5"]
    E, k, H, I, T, S = c["E"], c["k"], c["H"], c["I"], c["T"], c["S_variant"]
    base = synth.config_seed("c5")
    slab = synth.slab_bytes(synth.W_BF16, H, I)
    G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, 0), (E, H), c["sigma_g"], 1).view(np.int16)).cuda()
    warm = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_WARM, 0), (1024, H), 1.0, 1).view(np.int16)).cuda()
    wids = torch.empty((1024, k), dtype=torch.int32, device="cuda")
    ww = torch.empty((1024, k), dtype=torch.float32, device="cuda")
    m.moe_route(warm, 1, G, None, None, 1024, H, E, k, wids, ww, None)
    resident = torch.empty(S, dtype=torch.int32, device="cuda")
    m.cache_pick_static(wids, 1024 * k, E, S, resident)
    torch.cuda.synchronize()
    slots = store[torch.from_numpy(resident.cpu().numpy().astype(np.int64))].cuda()
    spec = dict(host_store=store, slot_store=slots, G=G, bias=None, resident=resident)
    nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_BF16, T_max=T, layers=[spec], n_threads=nthreads)
    xs = [torch.from_numpy(synth.normal(synth.key(base, synth.TAG_X, 0, st), (T, H), 1.0, 1).view(np.int16)).cuda()
          for st in range(2)]

    def timed(host_pass):
        nat.layer_step(0, xs[0], T, host_pass=host_pass)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            nat.layer_step(0, xs[1 - i % 2], T, host_pass=host_pass)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    auto_ms = timed(True)
    mode = nat.last_host_mode()
    nat.stats(reset=True)
    nat.layer_step(0, xs[0], T)
    hits, distinct, _, n_host = nat.stats(reset=True)
    nat.set_stream_threshold(-1)
    cpu_ms = timed(True)
    gpu_ms = timed(False)
    nat.close()
    return {"workload": "288-expert bf16 MoE layer, H=4096 I=1536 top-8, 2048 tokens, 144 experts resident, the "
                        f"other 144 in pinned host memory, native moe_layer_step, {nthreads} host threads",
            "tokens_per_s": round(T / auto_ms * 1e3, 1), "ms_per_step": round(auto_ms, 2),
            "host_misses_served_by": {1: "CPU lane", 2: "streamed through the GPU"}.get(mode, str(mode)),
            "hit_rate": round(hits / (T * k), 4), "host_experts_per_step": n_host,
            "streamed_gb_per_step": round(n_host * slab / 1e9, 3) if mode == 2 else 0,
            "cpu_lane": {"tokens_per_s": round(T / cpu_ms * 1e3, 1), "ms_per_step": round(cpu_ms, 2)},
            "gpu_only_ms_per_step": round(gpu_ms, 3)}


def bench_dynamic(m, torch, synth, SlotLayer, NativeStack, nthreads, link_gbs, steps=256, warmup=8):
    """128-expert W8A8 layer, Zipf(0.8) routing ids (permutation per layer),
    32 LRU slots starting empty, 256 steps of 16 tokens; x fresh per step.
    Timed with the native driver; the same steps are then replayed from
    Python from an empty cache again (the cache evolves identically) with HIP
    events around every cache_gather and moe_ffn_slots."""
    c = synth.CONFIGS["c3"]
    E, k, H, I, S, T = c["E"], c["k"], c["H"], c["I"], c["S"], c["T"]
    base = synth.config_seed("c3")
    slab = synth.slab_bytes(synth.W_W8A8, H, I)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    synth.slabs_into(store.data_ptr(), synth.W_W8A8, base, 0, 0, E, H, I, c["sigma_w"], slab)
    G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, 0), (E, H), c["sigma_g"], 1).view(np.int16)).cuda()
    ids_all = synth.zipf_ids(synth.key(base, synth.TAG_ZIPF_PERM), synth.key(base, synth.TAG_ZIPF_DRAW),
                             (warmup + steps) * T, E, k, c["zipf_s"])
    ids_all = torch.from_numpy(ids_all).cuda().reshape(warmup + steps, T * k)
    xs = torch.from_numpy(np.stack([synth.normal(synth.key(base, synth.TAG_X, 0, st), (T, H), 1.0, 1)
                                    for st in range(warmup + steps)]).view(np.int16)).cuda()
    spec = dict(host_store=store, slot_store=torch.empty((S, slab), dtype=torch.uint8, device="cuda"), G=G,
                bias=None, resident=None, policy="lru")
    elapsed = None
    for phase in ("warmup", "timed"):
        native = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_W8A8, T_max=T, layers=[spec],
                             n_threads=nthreads)  # a fresh, empty cache
        n = warmup if phase == "warmup" else steps
        off = 0 if phase == "warmup" else warmup
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            native.layer_step(0, xs[off + i], T, ids_in=ids_all[off + i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        hits, distinct, gathered, host = native.stats()
        native.close()
    # replay with events
    L = SlotLayer(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_W8A8, T_max=T, policy="lru", host_store=store,
                  slot_store=torch.empty((S, slab), dtype=torch.uint8, device="cuda"), G=G, n_threads=nthreads)
    L.init_cache(None)
    acc = torch.zeros(4, dtype=torch.int64, device="cuda")
    gev, fev = [], []
    for i in range(steps):
        L.gather_events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        L.ffn_events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        L.step(xs[warmup + i], T, ids_in=ids_all[warmup + i])
        acc += L.stats
        gev.append(L.gather_events)
        fev.append(L.ffn_events)
    torch.cuda.synchronize()
    L.gather_events = L.ffn_events = None
    assert [int(v) for v in acc.cpu()] == [hits, distinct, gathered, host], "replay differs from the timed run"
    g_ms = float(np.sum([a.elapsed_time(b) for a, b in gev]))
    g_bytes = gathered * slab
    g_gbs = g_bytes / (g_ms * 1e-3) / 1e9 if g_ms > 0 else None
    out = {"workload": "128-expert W8A8 MoE layer, H=2048 I=768 top-8, Zipf(0.8) ids, 32 LRU slots from empty, "
                       f"{steps} steps x {T} tokens, host pass on {nthreads} threads, native moe_layer_step",
           "tokens_per_s": round(T * steps / elapsed, 1), "ms_per_step": round(elapsed / steps * 1e3, 4),
           "hit_rate": round(hits / (steps * T * k), 4), "distinct_per_step": round(distinct / steps, 2),
           "gathered_per_step": round(gathered / steps, 2), "host_experts_per_step": round(host / steps, 2),
           "gather_gbs": None if g_gbs is None else round(g_gbs, 2),
           "gather_link_frac": None if (g_gbs is None or not link_gbs) else round(g_gbs / link_gbs, 4),
           "gather_bytes_per_step": int(g_bytes / steps),
           "ffn_ms": round(float(np.mean([a.elapsed_time(b) for a, b in fev])), 4)}
    return out


def bench_stack(m, torch, synth, SlotStack, NativeStack, nthreads, args, n_base=4):
    """The 48-layer stack of 512-expert top-10 layers (hidden 2048,
    intermediate 512) with 4-bit block weights (43.5 GB pinned host store),
    192 hot experts per layer resident in VRAM (16.3 GB), graded bias with
    cap -1 from per-layer Dirichlet(0.3) brightness.  Layers 0..3 draw their
    weights from the seeded generator; layer l >= 4 holds the experts of layer
    l % 4 in a per-layer permuted order (distinct memory per layer, same
    weight distribution) to keep set-up within a minute."""
    c = synth.CONFIGS["c4"]
    E, k, H, I, S, NL = c["E"], c["k"], c["H"], c["I"], c["S"], c["layers"]
    base = synth.config_seed("c4")
    slab = synth.slab_bytes(synth.W_Q4B32, H, I)
    t_setup = time.perf_counter()
    bases = [synth.slabs(synth.W_Q4B32, base, l, 0, E, H, I, c["sigma_w"]) for l in range(n_base)]
    specs = []
    for l in range(NL):
        b = synth.dirichlet(synth.key(base, synth.TAG_B, l), E, c["alpha"])
        resident = np.lexsort((np.arange(E), -b))[:S].astype(np.int32)
        hs = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
        if l < n_base:
            hs.numpy()[:] = bases[l]
        else:
            hs.numpy()[:] = bases[l % n_base][np.random.default_rng(1000 + l).permutation(E)]
        bias = torch.empty(E, dtype=torch.float32, device="cuda")
        m.moe_bias_table(torch.from_numpy(b).cuda(), E, S, c["cap"], bias)
        G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, l), (E, H), c["sigma_g"], 1)
                             .view(np.int16)).cuda()
        specs.append(dict(host_store=hs, slot_store=hs[torch.from_numpy(resident.astype(np.int64))].cuda(), G=G,
                          bias=bias, resident=torch.from_numpy(resident).cuda()))
    del bases
    stack = SlotStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_Q4B32, T_max=32, layers=specs, n_threads=nthreads)
    native = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_Q4B32, T_max=32, layers=specs, n_threads=nthreads)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    out = {"metric": "MoE-layer tokens/s; expert-weight HBM GB/s as % of peak; gather GB/s",
           "workload": "48 x 512-expert top-10 4-bit stack, H=2048 I=512, graded bias cap -1, 192 resident per "
                       f"layer, host pass on {nthreads} threads", "data": "synthetic", "setup_s": round(t_setup, 1),
           "host_store_gb": round(NL * E * slab / 1e9, 2), "slot_store_gb": round(NL * S * slab / 1e9, 2)}
    ids2 = torch.empty(32 * k, dtype=torch.int32, device="cuda")
    w2 = torch.empty(32 * k, dtype=torch.float32, device="cuda")
    for T, steps in ((1, args.stack_steps), (32, max(2, args.stack_steps // 2))):
        xs = [torch.from_numpy(synth.normal(synth.key(base, synth.TAG_X, 0, st), (T, H), 1.0, 1).view(np.int16))
              .cuda() for st in range(steps + 2)]
        for i in range(2):
            native.step(xs[i], T)
        torch.cuda.synchronize()
        native.stats(reset=True)
        t0 = time.perf_counter()
        for i in range(steps):
            native.step(xs[2 + i], T)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        n_hits, n_distinct, _, n_host = native.stats(reset=True)
        # replay of the same steps from Python (untimed): FFN events and the unbiased routing
        acc = torch.zeros(4, dtype=torch.int64, device="cuda")
        nob = torch.zeros(1, dtype=torch.int64, device="cuda")
        evs = []

        def on_layer(l, L, xl, y):
            acc.add_(L.stats)
            m.moe_route(xl, 1, L.G, None, None, T, H, E, k, ids2, w2, None)
            e2s = stack.states[l][1]
            nob.add_((e2s[ids2[:T * k].long()] >= 0).sum())

        for i in range(steps):
            stack.step(xs[2 + i], T, on_layer=on_layer, ffn_events=evs)
        torch.cuda.synchronize()
        hits, distinct, gathered, host = (int(v) for v in acc.cpu())
        assert (hits, distinct, host) == (n_hits, n_distinct, n_host), "replay differs from the timed steps"
        ffn_ms = float(np.sum([a.elapsed_time(b) for a, b in evs]))
        resident_slabs = distinct - host
        byts = resident_slabs * slab + steps * NL * T * H * 6
        picks = steps * NL * T * k
        out[f"T{T}"] = {"tokens_per_s": round(T * steps / elapsed, 2), "ms_per_step": round(elapsed / steps * 1e3, 3),
                        "driver": "native moe_stack_step",
                        "ffn_ms_per_step": round(ffn_ms / steps, 4),
                        "ffn_gbs": round(byts / (ffn_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(byts / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "hit_rate_with_bias": round(hits / picks, 4),
                        "hit_rate_without_bias": round(int(nob.item()) / picks, 4),
                        "resident_experts_per_layer": round(resident_slabs / (steps * NL), 2),
                        "host_experts_per_layer": round(host / (steps * NL), 2)}
    native.close()
    return out


def _drift(y, y0):
    """Relative L2 distance of a layer output from the unbiased layer's output."""
    return float((y - y0).double().norm()) / max(float(y0.double().norm()), 1e-30)


def bench_bias(m, torch, synth, SlotLayer, NativeStack, nthreads, steps=48, warmup=4):
    """Routing-bias variants of "Nudge, don't cut" on the same router.

    static: the 512-expert top-10 4-bit layer (hidden 2048, intermediate 512)
    with the 192 brightest experts of a Dirichlet(0.3) profile resident, 32
    tokens per step.  Variants: no bias; graded table (cap -1, -0.5); flat
    bias (-1, -0.75, -0.5); hard mask; graded cap -1 with damped weights.
    live: the 128-expert W8A8 layer (hidden 2048, intermediate 768, top-8)
    routed by its own router (gate ~N(0, 0.05)) through a 32-slot LRU cache
    from empty, 16 tokens per step, with live-cache affinity lambda in
    {0, 0.25, 0.5, 1}: the bias is rebuilt from the cache state before every
    step (moe_bias_affinity on the compute stream).
    Per variant: hit rate per routing id, experts served by the host per
    step (and gathered, live cache), layer tokens/s with the host pass on the
    native driver, and the layer-output drift: relative L2 distance of the
    variant's output from the unbiased layer's on the same tokens (the
    layer's output does not depend on what is cached, so the unbiased
    output is the same for every cache)."""
    out = {"workload": "routing-bias variants: static 512-expert top-10 4-bit layer, 192 hot resident, T=32; "
                       "live-cache affinity on a 128-expert W8A8 layer, 32 LRU slots, T=16",
           "data": "synthetic", "steps": steps}

    # ---------------------------------------------------------------- static cache
    c = synth.CONFIGS["c4"]
    E, k, H, I, S = c["E"], c["k"], c["H"], c["I"], c["S"]
    T = 32
    base = synth.config_seed("c4")
    slab = synth.slab_bytes(synth.W_Q4B32, H, I)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    synth.slabs_into(store.data_ptr(), synth.W_Q4B32, base, 0, 0, E, H, I, c["sigma_w"], slab)
    b = synth.dirichlet(synth.key(base, synth.TAG_B, 0), E, 0.3)
    resident = np.lexsort((np.arange(E), -b))[:S].astype(np.int32)
    res_t = torch.from_numpy(resident).cuda()
    slots = store[torch.from_numpy(resident.astype(np.int64))].cuda()
    G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, 0), (E, H), c["sigma_g"], 1).view(np.int16)).cuda()
    b_t = torch.from_numpy(b).cuda()
    xs = torch.from_numpy(np.stack([synth.normal(synth.key(base, synth.TAG_X, 0, 100 + i), (T, H), 1.0, 1)
                                    for i in range(warmup + steps)]).view(np.int16)).cuda()

    def table(kind, val):
        t = torch.empty(E, dtype=torch.float32, device="cuda")
        if kind == "graded":
            m.moe_bias_table(b_t, E, S, val, t)
        else:
            m.moe_bias_flat(b_t, E, S, val, t)
        return t

    variants = [("none", None, 0), ("graded cap -1", table("graded", -1.0), 0),
                ("graded cap -0.5", table("graded", -0.5), 0), ("flat -1", table("flat", -1.0), 0),
                ("flat -0.75", table("flat", -0.75), 0), ("flat -0.5", table("flat", -0.5), 0),
                ("hard mask", table("flat", -float("inf")), 0),
                ("graded cap -1, damped weights", table("graded", -1.0), m.MOE_ROUTE_DAMPED)]
    res_mask = torch.zeros(E, dtype=torch.bool, device="cuda")
    res_mask[res_t.long()] = True
    L = SlotLayer(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_Q4B32, T_max=T, policy="static", host_store=store,
                  slot_store=slots, G=G, n_threads=nthreads)
    L.init_cache(res_t)
    y0 = []
    rows = []
    for name, bias, flags in variants:
        # analysis pass: picks, hits and outputs through the Python-driven layer
        L.bias, L.route_flags = bias, flags
        hits, host_e, drift = 0, 0, []
        for i in range(steps):
            y = L.step(xs[warmup + i], T).clone()
            ids = L.ids[:T * k].long()
            hits += int(res_mask[ids].sum())
            host_e += int(torch.unique(ids[~res_mask[ids]]).numel())
            if name == "none":
                y0.append(y)
            else:
                drift.append(_drift(y, y0[i]))
        row = {"variant": name, "hit_rate": round(hits / (steps * T * k), 4),
               "host_experts_per_step": round(host_e / steps, 2),
               "output_drift": round(float(np.mean(drift)), 4) if drift else 0.0}
        if flags == 0:  # timing on the native driver (damped weights change no pick: the same work)
            nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_Q4B32, T_max=T, n_threads=nthreads,
                              layers=[dict(host_store=store, slot_store=slots, G=G, bias=bias, resident=res_t)])
            for i in range(warmup):
                nat.layer_step(0, xs[i], T)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                nat.layer_step(0, xs[warmup + i], T)
            torch.cuda.synchronize()
            row["tokens_per_s"] = round(T * steps / (time.perf_counter() - t0), 1)
            nat.close()
        rows.append(row)
    out["static"] = rows
    del L, slots, store

    # ---------------------------------------------------------------- live-cache affinity
    c = synth.CONFIGS["c3"]
    E, k, H, I, S = c["E"], c["k"], c["H"], c["I"], c["S"]
    T = c["T"]
    base = synth.config_seed("c3")
    slab = synth.slab_bytes(synth.W_W8A8, H, I)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    synth.slabs_into(store.data_ptr(), synth.W_W8A8, base, 0, 0, E, H, I, c["sigma_w"], slab)
    G = torch.from_numpy(synth.normal(synth.key(base, synth.TAG_G, 0), (E, H), c["sigma_g"], 1).view(np.int16)).cuda()
    xs = torch.from_numpy(np.stack([synth.normal(synth.key(base, synth.TAG_X, 0, 100 + i), (T, H), 1.0, 1)
                                    for i in range(warmup + steps)]).view(np.int16)).cuda()
    rows = []
    y0 = []
    for lam in (0.0, 0.25, 0.5, 1.0):
        bias = torch.zeros(E, dtype=torch.float32, device="cuda")
        L = SlotLayer(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_W8A8, T_max=T, policy="lru", host_store=store,
                      slot_store=torch.empty((S, slab), dtype=torch.uint8, device="cuda"), G=G, bias=bias,
                      n_threads=nthreads)
        L.init_cache(None)
        acc = torch.zeros(4, dtype=torch.int64, device="cuda")
        drift = []
        for i in range(warmup + steps):
            m.moe_bias_affinity(L.e2s, None, E, lam, bias)
            y = L.step(xs[i], T).clone()
            if i >= warmup:
                acc += L.stats
                if lam == 0.0:
                    y0.append(y)
                else:
                    drift.append(_drift(y, y0[i - warmup]))
        hits, distinct, gathered, host = [int(v) for v in acc.cpu()]
        row = {"lambda": lam, "hit_rate": round(hits / (steps * T * k), 4),
               "gathered_per_step": round(gathered / steps, 2), "host_experts_per_step": round(host / steps, 2),
               "output_drift": round(float(np.mean(drift)), 4) if drift else 0.0}
        # timing on the native driver, the affinity table rebuilt before each step on the same stream
        spec = dict(host_store=store, slot_store=torch.empty((S, slab), dtype=torch.uint8, device="cuda"), G=G,
                    bias=bias, resident=None, policy="lru")
        nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=synth.W_W8A8, T_max=T, layers=[spec], n_threads=nthreads)
        for i in range(warmup):
            m.moe_bias_affinity(nat.e2s(0), None, E, lam, bias)
            nat.layer_step(0, xs[i], T)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            m.moe_bias_affinity(nat.e2s(0), None, E, lam, bias)
            nat.layer_step(0, xs[warmup + i], T)
        torch.cuda.synchronize()
        row["tokens_per_s"] = round(T * steps / (time.perf_counter() - t0), 1)
        nat.close()
        rows.append(row)
        del L
    out["live_affinity"] = rows
    return out


def bench_replay(m, torch, synth, n_tok=4096, phase_len=256, every=500, s_zipf=0.8):
    """A routing trace replayed one decode token per step through the cache
    alone (cache_manage -> cache_gather, and for the repick policy
    cache_pick_static -> cache_repick -> cache_gather every `every` tokens),
    with real slab copies from the pinned store.  Layer shape and slab of the
    128-expert W8A8 layer (4.73 MB per expert), 32 slots, top-8.  The trace's
    popular handful changes: Zipf(0.8) over a permutation drawn anew for each
    phase of 256 tokens.  Policies: a static set from the first 500 tokens'
    picks; LRU and LFU from empty; the static set repicked every 500 tokens
    from the last 500 tokens' picks; and the perfect-foresight fixed set (the
    32 most-picked experts of the whole trace).  Reported per policy: hit
    rate per routing id, experts and bytes fetched while running (the initial
    upload of a static set is counted apart), and the GPU time of the replay."""
    c = synth.CONFIGS["c3"]
    E, k, H, I, S = c["E"], c["k"], c["H"], c["I"], c["S"]
    base = synth.config_seed("c3")
    slab = synth.slab_bytes(synth.W_W8A8, H, I)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    synth.slabs_into(store.data_ptr(), synth.W_W8A8, base, 0, 0, E, H, I, c["sigma_w"], slab)
    slots = torch.empty((S, slab), dtype=torch.uint8, device="cuda")
    trace = np.concatenate([synth.zipf_ids(synth.key(base, synth.TAG_ZIPF_PERM, 1, ph),
                                           synth.key(base, synth.TAG_ZIPF_DRAW, 1, ph),
                                           min(phase_len, n_tok - ph * phase_len), E, k, s_zipf)
                            for ph in range((n_tok + phase_len - 1) // phase_len)])
    trace_d = torch.from_numpy(trace).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    rows = []
    for name in ("static (first 500 tokens)", "lru", "lfu", f"repick every {every} tokens",
                 "perfect-foresight fixed set"):
        st_t = [torch.empty(E, **i32), torch.empty(S, **i32), torch.empty(S, **i32), torch.empty(S, **i32),
                torch.zeros(1, **i32)]
        st = m.cache_state(*st_t, E, S)
        policy = {"lru": m.MOE_LRU, "lfu": m.MOE_LFU}.get(name, m.MOE_STATIC)
        want = torch.empty(S, **i32)
        miss, n_miss = torch.empty(2 * S, **i32), torch.zeros(1, **i32)
        host_miss, n_host = torch.empty(E, **i32), torch.zeros(1, **i32)
        slot_ids = torch.empty(k, **i32)
        stats = torch.zeros(4, **i32)
        acc = torch.zeros(4, dtype=torch.int64, device="cuda")
        loads = torch.zeros(1, dtype=torch.int64, device="cuda")
        upload = 0
        if policy == m.MOE_STATIC:
            src = trace_d if name.startswith("perfect") else trace_d[:every]
            m.cache_pick_static(src.reshape(-1), src.numel(), E, S, want)
            m.cache_init(st, None)
            m.cache_repick(st, want, miss, n_miss)  # the upload at load time
            m.cache_gather(miss, n_miss, S, store, slots, slab)
            upload = S
        else:
            m.cache_init(st, None)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for t in range(n_tok):
            if name.startswith("repick") and t > 0 and t % every == 0:
                m.cache_pick_static(trace_d[t - every:t].reshape(-1), every * k, E, S, want)
                m.cache_repick(st, want, miss, n_miss)
                m.cache_gather(miss, n_miss, S, store, slots, slab)
                loads += n_miss
            m.cache_manage(st, policy, trace_d[t], k, slot_ids, miss, n_miss, host_miss, n_host, stats)
            if policy != m.MOE_STATIC:
                m.cache_gather(miss, n_miss, S, store, slots, slab)
            acc += stats
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        hits, distinct, gathered, host = [int(v) for v in acc.cpu()]
        fetched = gathered + int(loads.item())
        rows.append({"policy": name, "hit_rate": round(hits / (n_tok * k), 4), "experts_fetched": fetched,
                     "gb_fetched": round(fetched * slab / 1e9, 3), "upload_experts": upload,
                     "host_experts_per_token": round(host / n_tok, 3),
                     "gpu_ms_per_token": round(e0.elapsed_time(e1) / n_tok, 4),
                     "wall_ms_per_token": round(wall / n_tok * 1e3, 4)})
    return {"workload": f"routing trace of {n_tok} decode tokens (Zipf {s_zipf} over a permutation redrawn every "
                        f"{phase_len} tokens), 128 experts top-8, 32 slots of 4.73 MB (W8A8 slabs), cache only "
                        "(manage + gather, real copies)", "data": "synthetic", "policies": rows}


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
    # host link: pinned H2D copies of 1 GiB by the copy engine, ten of them
    del slots
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    src[::4096].fill_(3)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    link = 10 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"gbs": round(g_gbs, 2), "link_gbs": round(link, 2), "frac": round(g_gbs / link, 4),
            "slab_bytes": slab, "slabs_per_call": n, "link": "pinned hipMemcpyAsync H2D, 1 GiB x 10"}


def replicate(n):
    """n fresh processes of this benchmark with the same arguments (each with
    its own warm-up); one line: the first run's line with the median value and
    step time, and min / median / max of the headline figures over the runs."""
    import subprocess
    argv = []
    skip = False
    for a in sys.argv[1:]:
        if skip:
            skip = False
            continue
        if a == "--replicate":
            skip = True
            continue
        if a.startswith("--replicate="):
            continue
        argv.append(a)
    lines = []
    for i in range(n):
        r = subprocess.run([sys.executable, os.path.abspath(__file__)] + argv, stdout=subprocess.PIPE, text=True)
        if r.returncode != 0:
            sys.exit(r.returncode)
        lines.append(json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1]))
        print(f"run {i + 1}/{n}: {lines[-1].get('value')}", file=sys.stderr, flush=True)

    def stats(get):
        v = [get(d) for d in lines]
        v = [x for x in v if x is not None]
        return {"min": min(v), "median": float(np.median(v)), "max": max(v)} if v else None

    out = dict(lines[0])
    rep = {"runs": n, "value": stats(lambda d: d.get("value")), "ms_per_step": stats(lambda d: d.get("ms_per_step"))}
    if "roofline" in out:
        rep["roofline_frac"] = stats(lambda d: d["roofline"]["frac"])
    for leg, key in (("prefill", "ffn_ms"), ("gather", "frac"), ("dynamic", "tokens_per_s")):
        if isinstance(out.get(leg), dict) and key in out[leg]:
            rep[f"{leg}_{key}"] = stats(lambda d, leg=leg, key=key: d[leg][key])
    out["value"] = rep["value"]["median"]
    out["ms_per_step"] = rep["ms_per_step"]["median"]
    out["replicates"] = rep
    print(json.dumps(out), flush=True)


def cpu_baseline(synth, T, n_tok=48, reps=3):
    """The oracle (single-threaded C) on a bounded sample of the same workload:
    logits, top-k, weights and the full SwiGLU layer (every pick, resident or
    not) for n_tok tokens of the same layer, on one thread pinned to one core;
    the median of reps samples."""
    import oracle
    li = synth.LayerInputs("c2", T=n_tok)
    cpus = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {cpus[-1]})
    try:
        dts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            z = oracle.logits(li.x, li.x_dtype, li.G)
            ids = oracle.topk(z, li.k)
            w = oracle.route_weights(z, ids)
            oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids, w)
            dts.append(time.perf_counter() - t0)
    finally:
        os.sched_setaffinity(0, set(cpus))
    dt = float(np.median(dts))
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(n_tok / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_tok} tokens of the same layer: route + full SwiGLU layer in double, one thread pinned "
                      f"to one core, median of {reps} ({', '.join(f'{d:.1f}' for d in dts)} s)",
            "nproc": len(cpus), "cpu_model": model}


# ------------------------------------------------------------ HBM counters


def ffn_source_hash():
    """Hash of the FFN kernels' code: the sources with comments and
    whitespace taken out, so that only a change of the code itself voids the
    stored counter readings."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def profile_path(T):
    return os.path.join(PROFILE_DIR, f"moe_ffn_slots_bf16_decode_T{T}.txt")


def stored_traffic(T):
    """HBM bytes per moe_ffn_slots launch from the committed counter summary,
    or None when there is none for this batch or the kernels changed since."""
    p = profile_path(T)
    if not os.path.exists(p):
        return None
    rec = None
    with open(p) as fh:
        for line in fh:
            if line.startswith("record: "):
                rec = json.loads(line[len("record: "):])
    if not rec or rec.get("ffn_source_sha256") != ffn_source_hash() or rec.get("traffic_bytes_per_launch") is None:
        return None
    return rec["traffic_bytes_per_launch"]


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _short(name):
    n = name.split("(")[0] if "::" not in name else name
    for k in ("k_group_hist", "k_group_place", "k_group_small", "k_group", "k_gu", "k_down_tok", "k_down", "k_reduce16", "k_reduce",
              "k_manage_gather", "k_logits_mfma", "k_stream_chunk", "k_stream_pos", "k_route",
              "k_logits",
              "k_topk", "k_manage", "k_gather", "k_combine", "k_quant_rows", "k_block_sums", "k_pick_static",
              "k_bias_table", "k_cache_init", "k_pf_gemm", "k_pf_wide", "k_dec_gemm", "k_pf_tiles", "k_residual_bf16",
              "k_residual_f32"):
        if f"::{k}<" in name or f"::{k}(" in name:
            i = name.index(k)
            j = name.find("(", i)
            return name[i:j]
    return name[:60]


def _counter_per_dispatch(rows, counter):
    """{kernel short name: [per-dispatch value in KiB]} for one counter."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def _ffn_launches(rows, key, T=64):
    """Group per-dispatch rows into decode moe_ffn_slots launches of the
    batch T: each dispatch of its anchor kernel with the closest earlier and
    later kernels of its sequence (FFN_SEQS) by dispatch id.  Returns a list
    of {kernel short name: row}."""
    before, anchor, after = FFN_SEQS[T]
    by_id = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    names = [_short(r["Kernel_Name"]) for r in by_id]
    launches = []
    for i, nm in enumerate(names):
        if nm != anchor:
            continue
        got = {nm: by_id[i]}
        for want in before:
            for j in range(i - 1, max(-1, i - 8), -1):
                if names[j] == want:
                    got[want] = by_id[j]
                    break
        for want in after:
            for j in range(i + 1, min(len(names), i + 50)):
                if names[j] == want:
                    got[want] = by_id[j]
                    break
        if len(got) == 1 + len(before) + len(after):
            launches.append(got)
    return launches


def summarize(args):
    tr, fe, wr, cfe, cwr = args.summarize
    T = args.batch
    stats = _csv_rows(tr, "kernel_stats.csv")
    trace = _csv_rows(tr, "kernel_trace.csv")
    frows = [r for r in _csv_rows(fe, "counter_collection.csv") if r["Counter_Name"] == "FETCH_SIZE"]
    wrows = [r for r in _csv_rows(wr, "counter_collection.csv") if r["Counter_Name"] == "WRITE_SIZE"]
    cfetch = _counter_per_dispatch(_csv_rows(cfe, "counter_collection.csv"), "FETCH_SIZE")
    cwrite = _counter_per_dispatch(_csv_rows(cwr, "counter_collection.csv"), "WRITE_SIZE")

    def copy_kib(per):
        # the copy kernel is the only dispatch of --copy-calibration moving ~1 GiB
        vals = [v for vs in per.values() for v in vs if v > 100_000]
        return float(np.median(vals))

    gib_kib = (1 << 30) / 1024.0
    f_fetch = gib_kib / copy_kib(cfetch)   # bytes the counter misses per unit it reports
    f_write = gib_kib / copy_kib(cwrite)
    lines = []
    lines.append(f"rocprofv3 summary: moe_ffn_slots, bf16 decode layer (E=128 top-8, H=2048, I=768, T={T}, "
                 f"64 static slots)")
    lines.append("")
    if args.commands:
        lines.append("commands (run from the repository root on one MI355X; TMPDIR=/tmp):")
        with open(args.commands) as fh:
            lines.extend("  " + l.rstrip() for l in fh if l.strip())
        lines.append("")
    lines.append("kernel trace (--kernel-trace --stats), every kernel of the run (all benchmark legs):")
    lines.append(f"  {'kernel':<34}{'calls':>7}{'avg us':>10}{'min us':>10}{'max us':>10}")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:24]:
        lines.append(f"  {_short(r['Name']):<34}{int(r['Calls']):>7}{float(r['AverageNs']) / 1e3:>10.2f}"
                     f"{float(r['MinNs']) / 1e3:>10.2f}{float(r['MaxNs']) / 1e3:>10.2f}")
    lines.append("")
    launches = _ffn_launches(trace, "trace", T)
    per_k = {}
    for L in launches:
        for nm, r in L.items():
            per_k.setdefault(nm, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    seq = FFN_SEQS[T][0] + (FFN_SEQS[T][1],) + FFN_SEQS[T][2]
    lines.append(f"decode moe_ffn_slots launches found in the trace: {len(launches)} (each: "
                 f"{', '.join(seq)}, matched by dispatch id)")
    ffn_avg = 0.0
    for nm, v in per_k.items():
        lines.append(f"  {nm:<34}{np.mean(v):>10.2f} us")
        ffn_avg += float(np.mean(v))
    lines.append(f"  sum per launch (kernel time): {ffn_avg:.2f} us")
    lines.append("")
    lines.append(f"HBM counters per decode moe_ffn_slots launch (KiB per dispatch, mean over launches; "
                 f"calibration: a 1 GiB copy reads FETCH_SIZE {copy_kib(cfetch):.0f} KiB, WRITE_SIZE "
                 f"{copy_kib(cwrite):.0f} KiB, so factors {f_fetch:.3f} and {f_write:.3f}):")
    lines.append(f"  {'kernel':<34}{'FETCH KiB':>14}{'WRITE KiB':>14}{'scaled MB':>12}")
    fl, wl = _ffn_launches(frows, "fetch", T), _ffn_launches(wrows, "write", T)
    traffic = 0.0
    for nm in (fl[0].keys() if fl else []):
        fv = float(np.mean([float(L[nm]["Counter_Value"]) for L in fl]))
        wv = float(np.mean([float(L[nm]["Counter_Value"]) for L in wl])) if wl and nm in wl[0] else 0.0
        scaled = (fv * f_fetch + wv * f_write) * 1024
        traffic += scaled
        lines.append(f"  {nm:<34}{fv:>14.1f}{wv:>14.1f}{scaled / 1e6:>12.2f}")
    lines.append(f"  per launch (sum over its kernels): {traffic / 1e6:.2f} MB over {len(fl)} / {len(wl)} launches")
    rec = {"batch": T, "ffn_source_sha256": ffn_source_hash(), "ffn_kernels_avg_us": round(ffn_avg, 3),
           "launches": len(launches), "traffic_bytes_per_launch": int(traffic) if fl else None,
           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}
    lines.append("")
    lines.append("record: " + json.dumps(rec))
    out = args.out or profile_path(T)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def summarize_kernels(args):
    """Per kernel of a profiled run: calls, average duration, and HBM bytes
    per dispatch from FETCH_SIZE / WRITE_SIZE runs of the same command,
    scaled by what the counters read for a plain 1 GiB copy."""
    tr, fe, wr, cfe, cwr = args.summarize_kernels
    stats = _csv_rows(tr, "kernel_stats.csv")
    fetch = _counter_per_dispatch(_csv_rows(fe, "counter_collection.csv"), "FETCH_SIZE")
    write = _counter_per_dispatch(_csv_rows(wr, "counter_collection.csv"), "WRITE_SIZE")
    cfetch = _counter_per_dispatch(_csv_rows(cfe, "counter_collection.csv"), "FETCH_SIZE")
    cwrite = _counter_per_dispatch(_csv_rows(cwr, "counter_collection.csv"), "WRITE_SIZE")

    def copy_kib(per):
        return float(np.median([v for vs in per.values() for v in vs if v > 100_000]))

    gib_kib = (1 << 30) / 1024.0
    f_fetch, f_write = gib_kib / copy_kib(cfetch), gib_kib / copy_kib(cwrite)
    lines = [f"rocprofv3 summary: {args.title}", ""]
    if args.commands:
        lines.append("commands (run from the repository root on one MI355X; TMPDIR=/tmp):")
        with open(args.commands) as fh:
            lines.extend("  " + l.rstrip() for l in fh if l.strip())
        lines.append("")
    lines.append(f"HBM counters scaled by a 1 GiB copy: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f}; "
                 "per dispatch, mean over the kernel's dispatches")
    lines.append(f"  {'kernel':<34}{'calls':>7}{'avg us':>10}{'HBM MB':>10}{'GB/s':>9}")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:24]:
        nm = _short(r["Name"])
        us = float(r["AverageNs"]) / 1e3
        mb = None
        if nm in fetch:
            mb = (float(np.mean(fetch[nm])) * f_fetch + float(np.mean(write.get(nm, [0.0]))) * f_write) * 1024 / 1e6
        lines.append(f"  {nm:<34}{int(r['Calls']):>7}{us:>10.2f}" +
                     (f"{mb:>10.2f}{mb / us * 1e3:>9.0f}" if mb is not None else ""))
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {args.out}")


def summarize_prefill(args):
    """Per-kernel time, HBM counters and algorithmic bytes of the prefill legs
    (the 288-expert layer at 2048 and 16384 tokens) from the runs that
    --summarize reads.  A dispatch belongs to a leg by its grid (the 144-slot
    leg runs the same kernels on other grids): the GEMMs' grids are 8 XCDs x
    ceil(max tiles / 8) x column tiles workgroups of 256 threads, max tiles
    = min(S, P) + P / rows + 1 for tiles of 128 rows (2048 tokens) or 256
    (16384), as the library sizes those grids."""
    tr, fe, wr, cfe, cwr = args.summarize_prefill
    import synth
    c = synth.CONFIGS["c5"]
    E, k, H, I = c["E"], c["k"], c["H"], c["I"]
    trace = _csv_rows(tr, "kernel_trace.csv")
    frows = [r for r in _csv_rows(fe, "counter_collection.csv") if r["Counter_Name"] == "FETCH_SIZE"]
    wrows = [r for r in _csv_rows(wr, "counter_collection.csv") if r["Counter_Name"] == "WRITE_SIZE"]
    cfetch = _counter_per_dispatch(_csv_rows(cfe, "counter_collection.csv"), "FETCH_SIZE")
    cwrite = _counter_per_dispatch(_csv_rows(cwr, "counter_collection.csv"), "WRITE_SIZE")

    def copy_kib(per):
        return float(np.median([v for vs in per.values() for v in vs if v > 100_000]))

    gib_kib = (1 << 30) / 1024.0
    f_fetch, f_write = gib_kib / copy_kib(cfetch), gib_kib / copy_kib(cwrite)
    w_gu, w_dn = E * 2 * I * H * 2, E * H * I * 2  # every expert is resident and picked at both sizes
    legs = []
    for T in (2048, 16384):
        P = T * k
        big = T == 16384
        gu, dn = ("k_pf_wide<0>", "k_pf_wide<1>") if big else ("k_pf_gemm<0, 4>", "k_pf_gemm<1, 8>")
        tile_groups = (min(E, P) + P // (256 if big else 128) + 1 + 7) // 8
        # gate/up column tiles: 128 gate + up rows (wide tiles), 64 (128-row tiles, four 32-row blocks per wave)
        gu_cols = I // 128 if big else I // 64
        legs.append((T, [
            (gu, w_gu + T * H * 2 + P * I * 2, 2.0 * P * 2 * I * H, 8 * tile_groups * gu_cols * 256),
            (dn, w_dn + P * I * 2 + P * H * 2, 2.0 * P * H * I, 8 * tile_groups * (H // 256) * 256),
            ("k_reduce16", P * H * 2 + T * H * 4, 0.0, T * H // 8),
        ]))

    def pick(rows, name, grid, grid_key):
        out = []
        for r in rows:
            if _short(r["Kernel_Name"]) != name:
                continue
            if grid is not None and int(r[grid_key]) != grid:
                continue
            out.append(r)
        return out

    lines = ["rocprofv3 summary: moe_ffn_slots prefill legs, 288-expert bf16 layer (H=4096, I=1536, top-8, "
             "all experts resident) at 2048 and 16384 tokens", ""]
    if args.commands:
        lines.append("commands (run from the repository root on one MI355X; TMPDIR=/tmp):")
        with open(args.commands) as fh:
            lines.extend("  " + l.rstrip() for l in fh if l.strip())
        lines.append("")
    lines.append(f"HBM counters scaled by a 1 GiB copy: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f}. "
                 "Algorithmic bytes: weights once, activations in and out once (x, h, bf16 partials, y).")
    for T, ks in legs:
        # the leg's reductions: those dispatched right after its down GEMMs
        dn_ids = [int(r["Dispatch_Id"]) for r in pick(trace, ks[1][0], ks[1][3], "Grid_Size_X")]
        lines.append("")
        lines.append(f"{T} tokens ({T * k} picks):")
        lines.append(f"  {'kernel':<18}{'calls':>6}{'avg us':>10}{'HBM GB':>9}{'alg GB':>9}{'HBM/alg':>9}"
                     f"{'alg GB/s':>10}{'TFLOP/s':>9}")
        for name, alg, flops, grid in ks:
            tr_rows = pick(trace, name, None if grid is None else grid, "Grid_Size_X")
            f_rows = pick(frows, name, grid, "Grid_Size")
            w_rows = pick(wrows, name, grid, "Grid_Size")
            if name.startswith("k_reduce") and dn_ids:
                tr_rows = [r for r in tr_rows if int(r["Dispatch_Id"]) - 1 in dn_ids]
            if not tr_rows:
                continue
            us = float(np.mean([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr_rows]))
            fv = float(np.mean([float(r["Counter_Value"]) for r in f_rows])) if f_rows else 0.0
            wv = float(np.mean([float(r["Counter_Value"]) for r in w_rows])) if w_rows else 0.0
            hbm = (fv * f_fetch + wv * f_write) * 1024
            tfs = f"{flops / us / 1e6:>9.1f}" if flops else f"{'':>9}"
            lines.append(f"  {name:<18}{len(tr_rows):>6}{us:>10.1f}{hbm / 1e9:>9.2f}{alg / 1e9:>9.2f}"
                         f"{hbm / alg:>9.2f}{alg / us / 1e3:>10.0f}{tfs}")
    if args.prefill_mfma:
        lines.extend(_prefill_mfma_lines(args.prefill_mfma, trace, legs, pick))
    out = args.out or os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                   "moe_ffn_slots_bf16_prefill_c5.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def _prefill_mfma_lines(d, trace, legs, pick):
    """MFMA counters of the prefill GEMMs: the matrix cores' busy share
    (MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (GRBM_GUI_ACTIVE
    of one XCD x SIMDs)), the shader clock those busy cycles were counted at
    (GRBM_GUI_ACTIVE of one XCD / kernel time, the XCD's count recovered from
    MfmaUtil), and the bf16 flops the MFMA instructions did (MOPS x 512)
    against the algorithmic flops (the difference is the padding of partial
    tiles)."""
    rows = _csv_rows(d, "counter_collection.csv")
    simds = 4 * 256

    def per(name, counter, grid):
        v = [float(r["Counter_Value"]) for r in pick(rows, name, grid, "Grid_Size") if r["Counter_Name"] == counter]
        return float(np.mean(v)) if v else None

    out = ["", "MFMA counters (a run of its own: --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE MfmaUtil "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16), per call. MFMA busy: the matrix cores' busy share of the kernel's cycles "
           "(rocprofv3's MfmaUtil); clock: those cycles over the kernel time; MFMA TFLOP: the bf16 work the MFMA "
           "instructions did (tile padding included), alg TFLOP: 2 flops per multiply-add of the picks' rows; "
           "of peak: alg TFLOP/s over 2.5 PFLOP/s (2.4 GHz), at clock: over the peak at the measured clock:"]
    for T, ks in legs:
        out.append(f"  {T} tokens:")
        out.append(f"    {'kernel':<18}{'MFMA busy':>10}{'clock GHz':>10}{'MFMA TFLOP':>11}{'alg TFLOP':>10}"
                   f"{'MFMA/alg':>9}{'TFLOP/s':>9}{'of peak':>8}{'at clock':>9}")
        for name, alg, flops, grid in ks:
            if not flops:
                continue
            busy, gui, util, mops = (per(name, c, grid) for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                                                                   "MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
            tr_rows = pick(trace, name, grid, "Grid_Size_X")
            if None in (busy, util, mops) or not tr_rows or util <= 0:
                continue
            us = float(np.mean([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr_rows]))
            gui_one = busy * 100.0 / (util * simds)  # GRBM_GUI_ACTIVE of one XCD
            ghz = gui_one / us / 1e3
            mf = mops * 512
            tfs = flops / us / 1e6
            peak_at_clock = 2500.0 * ghz / 2.4
            out.append(f"    {name:<18}{util:>9.1f}%{ghz:>10.2f}{mf / 1e12:>11.2f}{flops / 1e12:>10.2f}"
                       f"{mf / flops:>9.2f}{tfs:>9.1f}{tfs / 2500.0:>8.3f}{tfs / peak_at_clock:>9.3f}")
    return out


if __name__ == "__main__":
    main()

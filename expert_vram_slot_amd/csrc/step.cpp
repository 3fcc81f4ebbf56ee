// Native driver of one expert-slot layer step, and of a stack of such layers
// joined by a residual stream: the entry points of moe_slot.h issued in the
// order the method needs them, with no interpreter between the calls.
//
// sozai.app transcript "rtx-3060-run-35b-llamacpp", "Full Transcript": all the
// GPU work of a layer runs as one unbroken sequence and the experts that stay
// in RAM are run by the CPU meanwhile; one add joins the two.  "Porting
// vllm-expert-cache to NVIDIA GPUs", "What this package does": manage, gather
// and remap come before the expert FFN, which runs in slot space.
//
//   compute  [x -> host]  moe_route -> cache_manage_gather -> moe_ffn_slots
//                                       (the cache step, the gather and the doorbell in one launch; without
//                                        a host pass: cache_manage [-> cache_gather])
//                                                       -> y_host -> moe_combine [-> moe_residual]
//   copy     x -> host (pinned)
//   caller's CPU thread               waits for the doorbell (the picks mirrored to pinned memory behind it),
//                                     then moe_ffn_host_misses, only when the step has host misses; when the
//                                     step gathered, checks that no copying workgroup gave up
#include <hip/hip_runtime.h>
#include <immintrin.h>
#include <string.h>

#include <chrono>

#include <new>

#include "stream.hpp"

struct moe_step {
    int T_max, E, k, H, I, S, w_type, x_dtype;
    size_t slab_bytes, ffn_ws_bytes;
    // device
    int32_t* meta;  // [3][T_max * k] picks, slots, weights, then 4 cache counters (one copy to the host)
    float* logits;  // [T_max][E]
    int32_t *miss, *n_miss, *host_miss, *n_host;
    void* ffn_ws;
    float *y, *y_host_dev;
    void* xbuf[2];  // residual stream of a stack
    int32_t* sync;  // [2] hand-off word of the fused cache step
    // pinned host
    void* h_x;
    int32_t* h_meta;  // [3][T_max * k] picks, slots, weights mirrored by the fused cache step
    float* h_y;
    moe_doorbell* bell;
    int32_t seq;  // sequence number of the last fused cache step
    hipEvent_t ev_x, ev_copy, ev_cache;
    int64_t stats_sum[4];  // cache counters summed over host-pass steps
    // streamed miss pass (batches of T_max >= kStreamMinT): a ring of 2 * R staging slots
    int ring_R;             // staging slots per half (0: no ring)
    void* ring;             // device [2R][slab_bytes]
    int32_t* s_pos;         // device [P_max]: position of a pick's expert in host_miss, or -1
    int32_t* s_cmiss;       // device [2][2R]: gather list of a chunk per half
    int32_t* s_ncmiss;      // device [2] (16 B apart)
    int32_t* s_cslots;      // device [2][P_max]: staging slot per pick of a chunk per half
    hipEvent_t ev_k[2], ev_g[2];
    int stream_min;         // picks per host expert from which a step streams (< 0: never)
    int last_mode;          // 0: no host misses, 1: CPU lane, 2: streamed
};

namespace {

constexpr int kBellTimeoutS = 10;  // seconds a layer step waits for its cache step's doorbell
// Streamed miss pass: a step of T_max >= kStreamMinT tokens gets a ring of 2 * kStreamR staging slots.  It
// streams its misses instead of running the CPU lane when the host picks reach kStreamPicks per host expert:
// measured on the 288-expert bf16 layer (144 resident, 16 host threads), the CPU lane took 24 / 31 / 68 / 90 /
// 99 / 106 / 125 / 133 ms at 256 / 512 / 1024 / 1280 / 1408 / 1536 / 1792 / 2048 tokens (7 / 14 / 28 / 36 / 39 /
// 43 / 50 / 57 picks per host expert) and the streamed pass 101-104 ms (the 144 slabs over the host link), so
// the two cost the same near 41 picks per expert.
constexpr int kStreamMinT = 128;
constexpr int kStreamR = 8;
constexpr int kStreamPicks = 40;

int hip_fail(const char* what, hipError_t e) {
    (void)hipGetLastError();
    return moe_fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

void release(moe_step* h) {
    if (!h) return;
    void* dev[] = {h->meta, h->logits, h->miss, h->n_miss, h->host_miss, h->n_host, h->ffn_ws,
                   h->y, h->y_host_dev, h->xbuf[0], h->xbuf[1], h->sync, h->ring, h->s_pos, h->s_cmiss,
                   h->s_ncmiss, h->s_cslots};
    for (void* p : dev)
        if (p) (void)hipFree(p);
    void* host[] = {h->h_x, h->h_meta, h->h_y, h->bell};
    for (void* p : host)
        if (p) (void)hipHostFree(p);
    hipEvent_t evs[] = {h->ev_x, h->ev_copy, h->ev_cache, h->ev_k[0], h->ev_k[1], h->ev_g[0], h->ev_g[1]};
    for (hipEvent_t e : evs)
        if (e) (void)hipEventDestroy(e);
    delete h;
}

}  // namespace

extern "C" {

moe_step* moe_step_create(int T_max, int E, int k, int H, int I, int S, int w_type) {
    if (T_max < 1 || E < 1 || k < 1 || k > E || H < 1 || I < 1 || S < 0 || S > E) {
        moe_fail(MOE_E_ARG, "moe_step_create: T_max=%d E=%d k=%d H=%d I=%d S=%d out of range", T_max, E, k, H, I, S);
        return nullptr;
    }
    moe_slab_layout_t lay;
    if (moe_slab_layout(w_type, H, I, &lay)) return nullptr;
    moe_step* h = new (std::nothrow) moe_step();
    if (!h) {
        moe_fail(MOE_E_NOMEM, "moe_step_create: out of host memory");
        return nullptr;
    }
    h->T_max = T_max;
    h->E = E;
    h->k = k;
    h->H = H;
    h->I = I;
    h->S = S;
    h->w_type = w_type;
    h->x_dtype = w_type == MOE_W_F32 ? MOE_X_F32 : MOE_X_BF16;
    h->slab_bytes = (size_t)((lay.total + 15) / 16 * 16);
    const size_t P = (size_t)T_max * k;
    const size_t xb = h->x_dtype == MOE_X_F32 ? 4 : 2;
    const int Sw = S > 0 ? S : 1;
    h->ring_R = T_max >= kStreamMinT ? kStreamR : 0;
    h->stream_min = kStreamPicks;
    // the FFN over the staging ring uses the same workspace (2R slots)
    h->ffn_ws_bytes = moe_ffn_workspace_bytes(T_max, k, Sw > 2 * h->ring_R ? Sw : 2 * h->ring_R, w_type, H, I);
    struct {
        void** p;
        size_t n;
    } dev[] = {{(void**)&h->meta, 12 * P + 16},
               {(void**)&h->logits, 4 * (size_t)T_max * E},
               {(void**)&h->miss, 8 * (size_t)Sw},
               {(void**)&h->n_miss, 16},
               {(void**)&h->host_miss, 4 * (size_t)E},
               {(void**)&h->n_host, 16},
               {&h->ffn_ws, h->ffn_ws_bytes},
               {(void**)&h->y, 4 * (size_t)T_max * H},
               {(void**)&h->y_host_dev, 4 * (size_t)T_max * H},
               {&h->xbuf[0], xb * T_max * H},
               {&h->xbuf[1], xb * T_max * H},
               {(void**)&h->sync, 16},
               {&h->ring, h->ring_R ? 2 * (size_t)h->ring_R * h->slab_bytes : 0},
               {(void**)&h->s_pos, h->ring_R ? 4 * P : 0},
               {(void**)&h->s_cmiss, h->ring_R ? 16 * (size_t)h->ring_R : 0},
               {(void**)&h->s_ncmiss, h->ring_R ? (size_t)32 : 0},
               {(void**)&h->s_cslots, h->ring_R ? 8 * P : 0}};
    for (auto& d : dev) {
        if (d.n == 0) continue;
        hipError_t e = hipMalloc(d.p, d.n);
        if (e != hipSuccess) {
            hip_fail("moe_step_create: hipMalloc", e);
            release(h);
            return nullptr;
        }
    }
    struct {
        void** p;
        size_t n;
    } host[] = {{&h->h_x, xb * T_max * H},
                {(void**)&h->h_meta, 12 * P + 16},
                {(void**)&h->h_y, 4 * (size_t)T_max * H},
                {(void**)&h->bell, sizeof(moe_doorbell)}};
    for (auto& d : host) {
        hipError_t e = hipHostMalloc(d.p, d.n, hipHostMallocDefault);
        if (e != hipSuccess) {
            hip_fail("moe_step_create: hipHostMalloc", e);
            release(h);
            return nullptr;
        }
    }
    hipError_t me = hipMemset(h->sync, 0, 16);
    if (me != hipSuccess) {
        hip_fail("moe_step_create: hipMemset", me);
        release(h);
        return nullptr;
    }
    memset(h->bell, 0, sizeof(moe_doorbell));
    h->seq = 0;
    hipEvent_t* evs[] = {&h->ev_x, &h->ev_copy, &h->ev_cache, &h->ev_k[0], &h->ev_k[1], &h->ev_g[0], &h->ev_g[1]};
    for (hipEvent_t* e : evs) {
        hipError_t r = hipEventCreateWithFlags(e, hipEventDisableTiming);
        if (r != hipSuccess) {
            hip_fail("moe_step_create: hipEventCreate", r);
            release(h);
            return nullptr;
        }
    }
    moe_ok();
    return h;
}

void moe_step_destroy(moe_step* h) { release(h); }

const float* moe_step_output(const moe_step* h) { return h ? h->y : nullptr; }

int moe_step_stats(moe_step* h, int64_t* out, int reset) {
    if (!h || !out) return moe_fail(MOE_E_ARG, "moe_step_stats: NULL argument");
    memcpy(out, h->stats_sum, sizeof(h->stats_sum));
    if (reset) memset(h->stats_sum, 0, sizeof(h->stats_sum));
    return moe_ok();
}

namespace {

// The streamed miss pass: the n_host non-resident experts of the step go to
// the GPU in chunks of R through the two halves of the staging ring.  Chunk
// c + 1's gather (side stream) is queued before chunk c's FFN (compute
// stream), so it runs while that FFN does; a half is gathered into again only
// after the FFN that read it (its index kernel is queued on the compute
// stream after that FFN, and the gather waits for the index kernel).  Each
// chunk's FFN result is added to y.
int stream_misses(moe_step* h, const moe_layer_desc* L, const void* x, int T, int n_host, float* y, hipStream_t s0,
                  hipStream_t s_side) {
    const int P = T * h->k, Pm = h->T_max * h->k, R = h->ring_R;
    const int32_t* ids = h->meta;
    const int32_t* slot_ids = h->meta + Pm;
    const float* w = reinterpret_cast<const float*>(h->meta + 2 * Pm);
    int rc;
    hipError_t e;
    if ((rc = moe_stream_pos(ids, slot_ids, P, h->host_miss, h->n_host, h->s_pos, s0))) return rc;
    const int nc = (n_host + R - 1) / R;
    auto issue_gather = [&](int c) -> int {
        const int b = c & 1;
        int32_t* cmiss = h->s_cmiss + b * 2 * R;
        int32_t* ncm = h->s_ncmiss + 4 * b;
        int r = moe_stream_chunk(h->s_pos, P, h->host_miss, h->n_host, c * R, R, b * R, cmiss, ncm,
                                 h->s_cslots + (size_t)b * Pm, s0);
        if (r) return r;
        hipError_t er;
        if ((er = hipEventRecord(h->ev_k[b], s0)) != hipSuccess) return hip_fail("moe_layer_step: event", er);
        if ((er = hipStreamWaitEvent(s_side, h->ev_k[b], 0)) != hipSuccess) return hip_fail("moe_layer_step: wait", er);
        if ((r = cache_gather(cmiss, ncm, R, L->host_store, h->ring, L->slab_bytes, s_side))) return r;
        if ((er = hipEventRecord(h->ev_g[b], s_side)) != hipSuccess) return hip_fail("moe_layer_step: event", er);
        return MOE_OK;
    };
    if ((rc = issue_gather(0))) return rc;
    for (int c = 0; c < nc; ++c) {
        const int b = c & 1;
        if (c + 1 < nc && (rc = issue_gather(c + 1))) return rc;
        if ((e = hipStreamWaitEvent(s0, h->ev_g[b], 0)) != hipSuccess) return hip_fail("moe_layer_step: wait", e);
        if ((rc = moe_ffn_slots(x, h->x_dtype, h->s_cslots + (size_t)b * Pm, w, T, h->k, h->ring, L->slab_bytes,
                                2 * R, h->w_type, h->H, h->I, h->y_host_dev, h->ffn_ws, h->ffn_ws_bytes, s0)))
            return rc;
        if ((rc = moe_combine(y, h->y_host_dev, T, h->H, s0))) return rc;
    }
    return MOE_OK;
}

// After the fused cache step of a step that gathered: wait for its kernel
// (normally finished long before) and read the doorbell's err word, set by a
// copying workgroup that gave up waiting for the managing one.
int check_gather(moe_step* h) {
    hipError_t e = hipEventSynchronize(h->ev_cache);
    if (e != hipSuccess) return hip_fail("moe_layer_step: wait for the cache step", e);
    if (__atomic_load_n(&h->bell->err, __ATOMIC_ACQUIRE) != 0)
        return moe_fail(MOE_E_HIP,
                        "moe_layer_step: a copying workgroup of the cache step gave up waiting for the managing one; "
                        "the gather of this step is incomplete (slot store and cache state disagree: cache_init "
                        "the layer again)");
    return MOE_OK;
}

}  // namespace

int moe_step_set_stream_threshold(moe_step* h, int picks_per_expert) {
    if (!h) return moe_fail(MOE_E_ARG, "moe_step_set_stream_threshold: NULL step");
    h->stream_min = picks_per_expert;
    return moe_ok();
}

int moe_step_last_host_mode(const moe_step* h) { return h ? h->last_mode : -1; }

int moe_layer_step(moe_step* h, const moe_layer_desc* L, const void* x, int T, const int32_t* ids_in, int host_pass,
                   int n_threads, float* y_out, hipStream_t s0, hipStream_t s_side, hipStream_t s_copy) {
    if (!h || !L || !x) return moe_fail(MOE_E_ARG, "moe_layer_step: NULL argument");
    if (T < 0 || T > h->T_max) return moe_fail(MOE_E_SHAPE, "moe_layer_step: T=%d outside [0, %d]", T, h->T_max);
    if (L->state.E != h->E || L->state.S != h->S || L->slab_bytes < h->slab_bytes)
        return moe_fail(MOE_E_SHAPE, "moe_layer_step: layer (E=%d, S=%d, slab %zu) does not match the step (E=%d, S=%d)",
                        L->state.E, L->state.S, L->slab_bytes, h->E, h->S);
    if (T == 0) return moe_ok();
    h->last_mode = 0;
    const int P = T * h->k, Pm = h->T_max * h->k;
    const size_t xbytes = (size_t)T * h->H * (h->x_dtype == MOE_X_F32 ? 4 : 2);
    float* y = y_out ? y_out : h->y;
    int32_t* ids = h->meta;
    int32_t* slot_ids = h->meta + Pm;
    float* w = reinterpret_cast<float*>(h->meta + 2 * Pm);
    hipError_t e;
    int rc;
    if (host_pass) {  // the host pass's activations leave while the router runs
        if ((e = hipEventRecord(h->ev_x, s0)) != hipSuccess) return hip_fail("moe_layer_step: event", e);
        if ((e = hipStreamWaitEvent(s_copy, h->ev_x, 0)) != hipSuccess) return hip_fail("moe_layer_step: wait", e);
        if ((e = hipMemcpyAsync(h->h_x, x, xbytes, hipMemcpyDeviceToHost, s_copy)) != hipSuccess)
            return hip_fail("moe_layer_step: x to host", e);
        if ((e = hipEventRecord(h->ev_copy, s_copy)) != hipSuccess) return hip_fail("moe_layer_step: event", e);
    }
    if (ids_in) {
        if ((e = hipMemcpyAsync(ids, ids_in, (size_t)P * 4, hipMemcpyDeviceToDevice, s0)) != hipSuccess)
            return hip_fail("moe_layer_step: given picks", e);
    }
    if ((rc = moe_route(x, h->x_dtype, L->G, L->bias, ids_in ? ids : nullptr, T, h->H, h->E, h->k, ids, w, h->logits,
                        s0)))
        return rc;
    const bool dynamic = L->policy != MOE_STATIC && h->S > 0;
    int32_t seq = 0;
    if (host_pass) {
        // one launch: the cache step, the gather of the misses, and the picks mirrored to
        // pinned memory behind a doorbell; err is cleared here, before the launch, because
        // only the kernel's copying workgroups ever set it
        seq = ++h->seq;
        h->bell->err = 0;
        if ((rc = cache_manage_gather(&L->state, L->policy, ids, P, w, slot_ids, h->miss, h->n_miss, h->host_miss,
                                      h->n_host, h->meta + 3 * Pm, L->host_store, L->slot_store, L->slab_bytes,
                                      h->sync, seq, h->bell, h->h_meta, h->h_meta + Pm,
                                      reinterpret_cast<float*>(h->h_meta + 2 * Pm), s0)))
            return rc;
        if ((e = hipEventRecord(h->ev_cache, s0)) != hipSuccess) return hip_fail("moe_layer_step: event", e);
    } else {
        // no host waits at all: the cache step, then (dynamic cache) the gather, in stream order
        if ((rc = cache_manage(&L->state, L->policy, ids, P, slot_ids, h->miss, h->n_miss, h->host_miss, h->n_host,
                               h->meta + 3 * Pm, s0)))
            return rc;
        if (dynamic && (rc = cache_gather(h->miss, h->n_miss, h->S, L->host_store, L->slot_store, L->slab_bytes, s0)))
            return rc;
    }
    if ((rc = moe_ffn_slots(x, h->x_dtype, slot_ids, w, T, h->k, L->slot_store, L->slab_bytes, h->S > 0 ? h->S : 1,
                            h->w_type, h->H, h->I, y, h->ffn_ws, h->ffn_ws_bytes, s0)))
        return rc;
    if (!host_pass) return moe_ok();
    // the doorbell: the picks are on the host once it shows this step's seq
    const auto t0 = std::chrono::steady_clock::now();
    for (int n = 0; __atomic_load_n(&h->bell->seq, __ATOMIC_ACQUIRE) != seq; ++n) {
        _mm_pause();
        if ((n & 1023) == 1023 &&
            std::chrono::steady_clock::now() - t0 > std::chrono::seconds(kBellTimeoutS)) {
            hipError_t pe = hipStreamQuery(s0);
            return moe_fail(MOE_E_HIP, "moe_layer_step: no doorbell from the cache step after %d s (stream: %s)",
                            kBellTimeoutS, hipGetErrorString(pe));
        }
    }
    for (int i = 0; i < 4; ++i) h->stats_sum[i] += h->bell->stats[i];
    const bool gathered = h->bell->n_miss > 0;
    const int n_host = h->bell->n_host;
    if (n_host == 0) return gathered ? check_gather(h) : moe_ok();  // every pick resident: nothing to add
    if (h->ring_R && h->stream_min >= 0) {
        // large batch: stream the misses through the GPU instead of the CPU lane when they are
        // picked often enough that moving their weights costs less than computing them here
        int host_picks = 0;
        for (int i = 0; i < P; ++i) host_picks += h->h_meta[Pm + i] < 0;
        if ((int64_t)host_picks >= (int64_t)h->stream_min * n_host) {
            h->last_mode = 2;
            if ((rc = stream_misses(h, L, x, T, n_host, y, s0, s_side))) return rc;
            return gathered ? check_gather(h) : moe_ok();
        }
    }
    h->last_mode = 1;
    // the host pass on this thread, while the GPU runs the FFN
    if ((e = hipEventSynchronize(h->ev_copy)) != hipSuccess) return hip_fail("moe_layer_step: wait for x", e);
    const int32_t* h_ids = h->h_meta;
    const int32_t* h_slot = h->h_meta + Pm;
    const float* h_w = reinterpret_cast<const float*>(h->h_meta + 2 * Pm);
    if ((rc = moe_ffn_host_misses(h->h_x, h->x_dtype, h_ids, h_slot, h_w, T, h->k, L->host_store, L->slab_bytes, h->E,
                                  h->w_type, h->H, h->I, h->h_y, n_threads)))
        return rc;
    if ((e = hipMemcpyAsync(h->y_host_dev, h->h_y, (size_t)T * h->H * 4, hipMemcpyHostToDevice, s0)) != hipSuccess)
        return hip_fail("moe_layer_step: host result to device", e);
    if ((rc = moe_combine(y, h->y_host_dev, T, h->H, s0))) return rc;
    return gathered ? check_gather(h) : moe_ok();
}

int moe_stack_step(moe_step* h, const moe_layer_desc* layers, int n_layers, const void* x, int T, int host_pass,
                   int n_threads, void* x_out, hipStream_t s0, hipStream_t s_side, hipStream_t s_copy) {
    if (!h || !layers || n_layers < 1 || !x || !x_out) return moe_fail(MOE_E_ARG, "moe_stack_step: bad arguments");
    const void* cur = x;
    for (int l = 0; l < n_layers; ++l) {
        int rc = moe_layer_step(h, &layers[l], cur, T, nullptr, host_pass, n_threads, nullptr, s0, s_side, s_copy);
        if (rc) return rc;
        void* nxt = l + 1 == n_layers ? x_out : h->xbuf[l & 1];
        if ((rc = moe_residual(cur, h->x_dtype, h->y, nxt, T, h->H, s0))) return rc;
        cur = nxt;
    }
    return moe_ok();
}

}  // extern "C"

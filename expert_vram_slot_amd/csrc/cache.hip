// Expert-slot cache on gfx950: state init, static resident set, the per-step
// manager (victims + miss list + remap) and the host-to-slot gather.
//
// "Porting vllm-expert-cache to NVIDIA GPUs", section "What this package
// does": per MoE layer and step, a manage kernel picks victims among the
// slots the step does not need and emits a miss list, a gather kernel copies
// the missing experts from host memory into their slots, and routing ids are
// remapped to slot space.  Section "Prove it is correct before measuring":
// the manager is deterministic (no atomics, no order-dependent reduction) and
// the gather reads pinned host memory from the device in 16-byte units.
#include <atomic>

#include "common.hpp"

namespace {

using v4u = uint32_t __attribute__((ext_vector_type(4)));

constexpr int MANAGE_THREADS = 1024;

__global__ void __launch_bounds__(1024) k_cache_init(int32_t* __restrict__ e2s, int32_t* __restrict__ s2e,
                                                     uint32_t* __restrict__ last, uint32_t* __restrict__ freq,
                                                     uint32_t* __restrict__ step, int E, int S,
                                                     const int32_t* __restrict__ resident) {
    __shared__ int32_t m[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) m[e] = -1;
    __syncthreads();
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        int e = resident ? resident[s] : -1;
        if (e < 0 || e >= E) e = -1;  // entries outside [0, E) leave the slot empty
        s2e[s] = e;
        last[s] = 0;
        freq[s] = 0;
        if (e >= 0) m[e] = s;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) e2s[e] = m[e];
    if (threadIdx.x == 0) *step = 0;
}

// Static resident set: S most-picked experts, ties to the lower id.
__global__ void __launch_bounds__(1024) k_pick_static(const int32_t* __restrict__ ids, int n_ids, int E, int S,
                                                      int32_t* __restrict__ resident) {
    __shared__ int cnt[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    // integer counting: the totals do not depend on the order of the adds
    for (int i = threadIdx.x; i < n_ids; i += blockDim.x) {
        const int e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = cnt[e];
        int rank = 0;
        for (int o = 0; o < E; ++o) {
            const int co = cnt[o];
            rank += (co > c) || (co == c && o < e);
        }
        if (rank < S) resident[rank] = e;
    }
}

// Victim order: empty slots first; then LRU by last use, LFU by use count
// then last use; then the lower slot.
__device__ __forceinline__ bool victim_before(int policy, bool occ_a, uint32_t f_a, uint32_t l_a, int a, bool occ_b,
                                              uint32_t f_b, uint32_t l_b, int b) {
    if (occ_a != occ_b) return !occ_a;
    if (occ_a) {
        if (policy == MOE_LFU && f_a != f_b) return f_a < f_b;
        if (l_a != l_b) return l_a < l_b;
    }
    return a < b;
}

// One cache step in one workgroup of 1024 threads.
__device__ __forceinline__ void manage_core(int32_t* __restrict__ e2s, int32_t* __restrict__ s2e,
                                            uint32_t* __restrict__ last, uint32_t* __restrict__ freq,
                                            uint32_t* __restrict__ stepp, int E, int S, int policy,
                                            const int32_t* __restrict__ ids, int n_ids,
                                            int32_t* __restrict__ slot_ids, int32_t* __restrict__ miss,
                                            int32_t* __restrict__ n_miss, int32_t* __restrict__ host_miss,
                                            int32_t* __restrict__ n_host, int32_t* __restrict__ stats) {
    __shared__ int32_t me2s[MOE_MAX_E];
    __shared__ unsigned char need[MOE_MAX_E];
    __shared__ int32_t misses[MOE_MAX_E];
    __shared__ int32_t ms2e[MOE_MAX_S];
    __shared__ uint32_t mlast[MOE_MAX_S], mfreq[MOE_MAX_S];
    __shared__ unsigned char cand[MOE_MAX_S];
    __shared__ int32_t victim[MOE_MAX_S];
    __shared__ int scratch[MANAGE_THREADS / 64 + 1];

    const int tid = threadIdx.x;
    const uint32_t now = *stepp;
    const bool dynamic = policy != MOE_STATIC;

    for (int e = tid; e < E; e += MANAGE_THREADS) {
        me2s[e] = e2s[e];
        need[e] = 0;
    }
    __syncthreads();
    // needed experts; routing ids resident at entry
    int hits = 0;
    for (int i = tid; i < n_ids; i += MANAGE_THREADS) {
        const int e = ids[i];
        if (e < 0 || e >= E) continue;  // ids outside [0, E) are ignored (their slot_ids become -1)
        need[e] = 1;                    // every writer stores the same value
        hits += me2s[e] >= 0;
    }
    int hit_total;
    (void)moe::block_exclusive_scan(hits, scratch, &hit_total);

    // misses in ascending expert id; hits refresh their slot
    int n_all = 0, distinct = 0;
    for (int e0 = 0; e0 < E; e0 += MANAGE_THREADS) {
        const int e = e0 + tid;
        const bool nd = e < E && need[e];
        const bool ms = nd && me2s[e] < 0;
        int cnt, dcnt;
        const int pos = moe::block_exclusive_scan(ms ? 1 : 0, scratch, &cnt);
        (void)moe::block_exclusive_scan(nd ? 1 : 0, scratch, &dcnt);
        if (ms) misses[n_all + pos] = e;
        if (nd && !ms && dynamic) {
            const int s = me2s[e];
            last[s] = now;
            if (policy == MOE_LFU) freq[s] += 1;
        }
        n_all += cnt;
        distinct += dcnt;
    }
    __syncthreads();

    // victims: slots holding nothing needed, in victim order
    int n_cand = 0;
    if (dynamic) {
        for (int s = tid; s < S; s += MANAGE_THREADS) {
            const int o = s2e[s];
            ms2e[s] = o;
            mlast[s] = last[s];
            mfreq[s] = freq[s];
            cand[s] = (o < 0) || !need[o];
        }
        __syncthreads();
        int c_local = 0;
        for (int s = tid; s < S; s += MANAGE_THREADS) {
            if (!cand[s]) continue;
            ++c_local;
            const bool occ = ms2e[s] >= 0;
            int rank = 0;
            for (int o = 0; o < S; ++o)
                if (cand[o] && victim_before(policy, ms2e[o] >= 0, mfreq[o], mlast[o], o, occ, mfreq[s], mlast[s], s))
                    ++rank;
            victim[rank] = s;
        }
        (void)moe::block_exclusive_scan(c_local, scratch, &n_cand);
    }

    // the i-th miss takes the i-th victim; the rest go to the host pass
    const int n_g = n_all < n_cand ? n_all : n_cand;
    for (int i = tid; i < n_all; i += MANAGE_THREADS) {
        const int e = misses[i];
        if (i < n_g) {
            const int s = victim[i];
            const int old = ms2e[s];
            if (old >= 0) me2s[old] = -1;  // old experts are distinct and not needed
            me2s[e] = s;
            s2e[s] = e;
            last[s] = now;
            freq[s] = 1;
            miss[2 * i] = e;
            miss[2 * i + 1] = s;
        } else {
            host_miss[i - n_g] = e;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += MANAGE_THREADS) e2s[e] = me2s[e];
    for (int i = tid; i < n_ids; i += MANAGE_THREADS) {
        const int e = ids[i];
        slot_ids[i] = (e >= 0 && e < E) ? me2s[e] : -1;
    }
    if (tid == 0) {
        *n_miss = n_g;
        *n_host = n_all - n_g;
        *stepp = now + 1;
        if (stats) {
            stats[0] = hit_total;
            stats[1] = distinct;
            stats[2] = n_g;
            stats[3] = n_all - n_g;
        }
    }
}

__global__ void __launch_bounds__(MANAGE_THREADS) k_manage(int32_t* __restrict__ e2s, int32_t* __restrict__ s2e,
                                                           uint32_t* __restrict__ last, uint32_t* __restrict__ freq,
                                                           uint32_t* __restrict__ stepp, int E, int S, int policy,
                                                           const int32_t* __restrict__ ids, int n_ids,
                                                           int32_t* __restrict__ slot_ids, int32_t* __restrict__ miss,
                                                           int32_t* __restrict__ n_miss,
                                                           int32_t* __restrict__ host_miss,
                                                           int32_t* __restrict__ n_host, int32_t* __restrict__ stats) {
    manage_core(e2s, s2e, last, freq, stepp, E, S, policy, ids, n_ids, slot_ids, miss, n_miss, host_miss, n_host,
                stats);
}

// Periodic repick in one workgroup: the new set is the distinct valid
// experts of want[0..S); its members already resident keep their slots, the
// others take, in ascending expert id, the slots whose expert is not in the
// new set (empty ones included), in ascending slot order.  The loads are the
// miss list of the gather that follows.
__global__ void __launch_bounds__(MANAGE_THREADS) k_repick(int32_t* __restrict__ e2s, int32_t* __restrict__ s2e,
                                                           uint32_t* __restrict__ last, uint32_t* __restrict__ freq,
                                                           const uint32_t* __restrict__ stepp, int E, int S,
                                                           const int32_t* __restrict__ want,
                                                           int32_t* __restrict__ miss, int32_t* __restrict__ n_miss) {
    __shared__ int32_t me2s[MOE_MAX_E];
    __shared__ unsigned char in_new[MOE_MAX_E];
    __shared__ int32_t loads[MOE_MAX_S];
    __shared__ int32_t victim[MOE_MAX_S];
    __shared__ int scratch[MANAGE_THREADS / 64 + 1];
    const int tid = threadIdx.x;
    const uint32_t now = *stepp;
    for (int e = tid; e < E; e += MANAGE_THREADS) {
        me2s[e] = e2s[e];
        in_new[e] = 0;
    }
    __syncthreads();
    for (int i = tid; i < S; i += MANAGE_THREADS) {
        const int e = want[i];
        if (e >= 0 && e < E) in_new[e] = 1;  // every writer stores the same value
    }
    __syncthreads();
    int n_load = 0;
    for (int e0 = 0; e0 < E; e0 += MANAGE_THREADS) {
        const int e = e0 + tid;
        const bool ld = e < E && in_new[e] && me2s[e] < 0;
        int cnt;
        const int pos = moe::block_exclusive_scan(ld ? 1 : 0, scratch, &cnt);
        if (ld) loads[n_load + pos] = e;  // at most S members, so at most S loads
        n_load += cnt;
    }
    int n_vict = 0;
    for (int s0 = 0; s0 < S; s0 += MANAGE_THREADS) {
        const int s = s0 + tid;
        bool v = false;
        if (s < S) {
            const int o = s2e[s];
            v = o < 0 || !in_new[o];
        }
        int cnt;
        const int pos = moe::block_exclusive_scan(v ? 1 : 0, scratch, &cnt);
        if (v) victim[n_vict + pos] = s;
        n_vict += cnt;
    }
    __syncthreads();
    for (int i = tid; i < n_load; i += MANAGE_THREADS) {  // n_load <= n_vict
        const int e = loads[i], s = victim[i];
        const int old = s2e[s];
        if (old >= 0) me2s[old] = -1;  // old experts are distinct and leave the set
        me2s[e] = s;
        s2e[s] = e;
        last[s] = now;
        freq[s] = 0;
        miss[2 * i] = e;
        miss[2 * i + 1] = s;
    }
    __syncthreads();
    for (int e = tid; e < E; e += MANAGE_THREADS) e2s[e] = me2s[e];
    if (tid == 0) *n_miss = n_load;
}

// Copy slabs host -> slot.  The flattened (miss, 16-byte granule) space is
// walked grid-stride; each thread keeps UNROLL loads in flight so the host
// link sees many outstanding reads.
constexpr int GATHER_THREADS = 256;
constexpr int GATHER_UNROLL = 4;

__global__ void __launch_bounds__(GATHER_THREADS) k_gather(const int32_t* __restrict__ miss,
                                                           const int32_t* __restrict__ n_miss,
                                                           int max_miss, const unsigned char* __restrict__ host,
                                                           unsigned char* __restrict__ slots, uint64_t slab_bytes) {
    const uint64_t per = slab_bytes / 16;
    const int nm = min(max(*n_miss, 0), max_miss);  // never beyond the miss buffer
    const uint64_t total = (uint64_t)nm * per;
    const uint64_t stride = (uint64_t)gridDim.x * GATHER_THREADS * GATHER_UNROLL;
    for (uint64_t base = (uint64_t)blockIdx.x * GATHER_THREADS * GATHER_UNROLL + threadIdx.x; base < total;
         base += stride) {
        v4u v[GATHER_UNROLL];
        uint64_t dst[GATHER_UNROLL];
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const uint64_t c = base + (uint64_t)u * GATHER_THREADS;
            dst[u] = ~0ull;
            if (c < total) {
                const uint64_t m = c / per, g = c - m * per;
                const uint64_t e = (uint64_t)miss[2 * m], s = (uint64_t)miss[2 * m + 1];
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(host + e * slab_bytes) + g);
                dst[u] = s * slab_bytes + g * 16;
            }
        }
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u)
            if (dst[u] != ~0ull) *reinterpret_cast<v4u*>(slots + dst[u]) = v[u];
    }
}

// The copy loop of the gather over workgroups wg of nwg (blockDim threads each).
__device__ __forceinline__ void gather_core(const int32_t* __restrict__ miss, int nm,
                                            const unsigned char* __restrict__ host, unsigned char* __restrict__ slots,
                                            uint64_t slab_bytes, int wg, int nwg) {
    const uint64_t per = slab_bytes / 16;
    const uint64_t total = (uint64_t)nm * per;
    const uint64_t nth = blockDim.x;
    const uint64_t stride = (uint64_t)nwg * nth * GATHER_UNROLL;
    for (uint64_t base = (uint64_t)wg * nth * GATHER_UNROLL + threadIdx.x; base < total; base += stride) {
        v4u v[GATHER_UNROLL];
        uint64_t dst[GATHER_UNROLL];
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const uint64_t c = base + (uint64_t)u * nth;
            dst[u] = ~0ull;
            if (c < total) {
                const uint64_t m = c / per, g = c - m * per;
                const uint64_t e = (uint64_t)miss[2 * m], s = (uint64_t)miss[2 * m + 1];
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(host + e * slab_bytes) + g);
                dst[u] = s * slab_bytes + g * 16;
            }
        }
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u)
            if (dst[u] != ~0ull) *reinterpret_cast<v4u*>(slots + dst[u]) = v[u];
    }
}

// Polls of the hand-off word before a copying workgroup of the fused cache
// step gives up (moe_fused_spin_limit changes it; 0 makes every copying
// workgroup give up at once, which tests the reporting of that case).
std::atomic<uint32_t> g_fused_spin_limit{1u << 22};

// Fused cache step.  Workgroup 0 runs the cache step; its first wave then
// mirrors the picks to pinned host memory and rings the doorbell (system-scope
// release), and thread 0 releases the hand-off word (device scope).  The
// other workgroups wait for the hand-off (at most spin_max polls) and all of
// them copy the missing slabs.  A workgroup that stops waiting copies nothing
// and says so in sync[1] (device) and in the doorbell's err word (pinned host
// memory, system scope); both words are only ever set here, never cleared, so
// a late managing workgroup cannot hide the report.
__global__ void __launch_bounds__(MANAGE_THREADS) k_manage_gather(
    int32_t* __restrict__ e2s, int32_t* __restrict__ s2e, uint32_t* __restrict__ last, uint32_t* __restrict__ freq,
    uint32_t* __restrict__ stepp, int E, int S, int policy, const int32_t* __restrict__ ids, int n_ids,
    const float* __restrict__ w, int32_t* __restrict__ slot_ids, int32_t* __restrict__ miss,
    int32_t* __restrict__ n_miss, int32_t* __restrict__ host_miss, int32_t* __restrict__ n_host,
    int32_t* __restrict__ stats, const unsigned char* __restrict__ host, unsigned char* __restrict__ slots,
    uint64_t slab_bytes, int32_t* __restrict__ sync, int32_t seq, moe_doorbell* __restrict__ bell,
    int32_t* __restrict__ bell_ids, int32_t* __restrict__ bell_slots, float* __restrict__ bell_w, uint32_t spin_max) {
    __shared__ int ok;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        manage_core(e2s, s2e, last, freq, stepp, E, S, policy, ids, n_ids, slot_ids, miss, n_miss, host_miss, n_host,
                    stats);
        __threadfence();  // every wave's results in device memory before the hand-off below
        __syncthreads();
        if (tid < 64) {  // the first wave: mirror, then the doorbell
            if (bell_ids)
                for (int i = tid; i < n_ids; i += 64) bell_ids[i] = ids[i];
            if (bell_slots)
                for (int i = tid; i < n_ids; i += 64) bell_slots[i] = slot_ids[i];
            if (bell_w && w)
                for (int i = tid; i < n_ids; i += 64) bell_w[i] = w[i];
            if (bell) {
                if (tid == 0) {
                    bell->n_miss = *n_miss;
                    bell->n_host = *n_host;
                    for (int q = 0; q < 4; ++q) bell->stats[q] = stats ? stats[q] : 0;
                }
                __threadfence_system();  // every lane's mirror stores before the doorbell
                if (tid == 0) __hip_atomic_store(&bell->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
        if (tid == 0) __hip_atomic_store(&sync[0], seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        ok = 1;
    } else if (tid == 0) {
        int v = 0;
        uint32_t n = 0;
        for (; n < spin_max; ++n) {
            v = __hip_atomic_load(&sync[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if (v == seq) break;
            __builtin_amdgcn_s_sleep(2);
        }
        ok = v == seq;
        if (!ok) {
            atomicOr(&sync[1], 1);
            if (bell) __hip_atomic_store(&bell->err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    __syncthreads();
    if (!ok || policy == MOE_STATIC) return;
    const int nm = min(max(__hip_atomic_load(n_miss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0), S);
    gather_core(miss, nm, host, slots, slab_bytes, blockIdx.x, gridDim.x);
}

int check_state(const moe_cache_state* st, const char* who) {
    MOE_REQUIRE(st && st->e2s && st->s2e && st->last && st->freq && st->step, MOE_E_ARG,
                "%s: cache state and its arrays must be non-NULL", who);
    MOE_REQUIRE(st->E >= 1 && st->S >= 0, MOE_E_ARG, "%s: E=%d S=%d out of range", who, st->E, st->S);
    MOE_REQUIRE(st->E <= MOE_MAX_E && st->S <= MOE_MAX_S && st->S <= st->E, MOE_E_SHAPE,
                "%s: need S=%d <= E=%d, E <= %d, S <= %d", who, st->S, st->E, MOE_MAX_E, MOE_MAX_S);
    return MOE_OK;
}

}  // namespace

extern "C" {

int cache_init(const moe_cache_state* st, const int32_t* resident, hipStream_t stream) {
    int rc = check_state(st, "cache_init");
    if (rc) return rc;
    hipLaunchKernelGGL(k_cache_init, dim3(1), dim3(1024), 0, stream, st->e2s, st->s2e, st->last, st->freq, st->step,
                       st->E, st->S, resident);
    return moe_check_launch("cache_init");
}

int cache_pick_static(const int32_t* ids, int n_ids, int E, int S, int32_t* resident, hipStream_t stream) {
    MOE_REQUIRE(ids && resident && n_ids >= 0 && E >= 1 && S >= 0, MOE_E_ARG, "cache_pick_static: bad arguments");
    MOE_REQUIRE(E <= MOE_MAX_E && S <= E, MOE_E_SHAPE, "cache_pick_static: need S=%d <= E=%d <= %d", S, E, MOE_MAX_E);
    if (S == 0) return moe_ok();
    hipLaunchKernelGGL(k_pick_static, dim3(1), dim3(1024), 0, stream, ids, n_ids, E, S, resident);
    return moe_check_launch("cache_pick_static");
}

int cache_manage(const moe_cache_state* st, int policy, const int32_t* ids, int n_ids, int32_t* slot_ids,
                 int32_t* miss, int32_t* n_miss, int32_t* host_miss, int32_t* n_host, int32_t* stats,
                 hipStream_t stream) {
    int rc = check_state(st, "cache_manage");
    if (rc) return rc;
    MOE_REQUIRE(policy == MOE_STATIC || policy == MOE_LRU || policy == MOE_LFU, MOE_E_ARG,
                "cache_manage: unknown policy %d", policy);
    MOE_REQUIRE(n_ids >= 0 && n_ids <= (1 << 24), MOE_E_SHAPE, "cache_manage: n_ids=%d out of range", n_ids);
    MOE_REQUIRE((ids && slot_ids) || n_ids == 0, MOE_E_ARG, "cache_manage: ids and slot_ids must be non-NULL");
    MOE_REQUIRE(miss && n_miss && host_miss && n_host, MOE_E_ARG,
                "cache_manage: miss, n_miss, host_miss and n_host must be non-NULL");
    hipLaunchKernelGGL(k_manage, dim3(1), dim3(MANAGE_THREADS), 0, stream, st->e2s, st->s2e, st->last, st->freq,
                       st->step, st->E, st->S, policy, ids, n_ids, slot_ids, miss, n_miss, host_miss, n_host, stats);
    return moe_check_launch("cache_manage");
}

int cache_manage_gather(const moe_cache_state* st, int policy, const int32_t* ids, int n_ids, const float* w,
                        int32_t* slot_ids, int32_t* miss, int32_t* n_miss, int32_t* host_miss, int32_t* n_host,
                        int32_t* stats, const void* host_store, void* slot_store, size_t slab_bytes, int32_t* sync,
                        int32_t seq, moe_doorbell* bell, int32_t* bell_ids, int32_t* bell_slots, float* bell_w,
                        hipStream_t stream) {
    int rc = check_state(st, "cache_manage_gather");
    if (rc) return rc;
    MOE_REQUIRE(policy == MOE_STATIC || policy == MOE_LRU || policy == MOE_LFU, MOE_E_ARG,
                "cache_manage_gather: unknown policy %d", policy);
    MOE_REQUIRE(n_ids >= 0 && n_ids <= (1 << 24), MOE_E_SHAPE, "cache_manage_gather: n_ids=%d out of range", n_ids);
    MOE_REQUIRE((ids && slot_ids) || n_ids == 0, MOE_E_ARG, "cache_manage_gather: ids and slot_ids must be non-NULL");
    MOE_REQUIRE(miss && n_miss && host_miss && n_host && sync, MOE_E_ARG,
                "cache_manage_gather: miss, n_miss, host_miss, n_host and sync must be non-NULL");
    const unsigned char* dev_host = nullptr;
    int nwg = 1;
    if (policy != MOE_STATIC && st->S > 0) {
        MOE_REQUIRE(host_store && slot_store, MOE_E_ARG, "cache_manage_gather: host_store and slot_store needed");
        MOE_REQUIRE(slab_bytes > 0 && slab_bytes % 16 == 0 && moe_aligned16(host_store) && moe_aligned16(slot_store),
                    MOE_E_ALIGN, "cache_manage_gather: slab_bytes=%zu and both stores must be 16-byte aligned",
                    slab_bytes);
        void* dev = nullptr;
        hipError_t e = hipHostGetDevicePointer(&dev, const_cast<void*>(host_store), 0);
        if (e != hipSuccess || !dev) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_ARG, "cache_manage_gather: host_store is not pinned, device-visible host memory (%s)",
                            hipGetErrorString(e));
        }
        dev_host = reinterpret_cast<const unsigned char*>(dev);
        // copying workgroups: enough 16-byte loads in flight for the host link, and all co-resident
        const uint64_t chunks = (uint64_t)st->S * (slab_bytes / 16);
        const uint64_t want = (chunks + (uint64_t)MANAGE_THREADS * GATHER_UNROLL - 1) /
                              ((uint64_t)MANAGE_THREADS * GATHER_UNROLL);
        nwg = (int)(want < 1 ? 1 : want > 128 ? 128 : want);
    }
    // device addresses of the pinned doorbell and mirrors, looked up on every call
    void* dptr[4] = {bell, bell_ids, bell_slots, bell_w};
    for (void*& q : dptr) {
        if (!q) continue;
        void* d = nullptr;
        hipError_t e = hipHostGetDevicePointer(&d, q, 0);
        if (e != hipSuccess || !d) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_ARG, "cache_manage_gather: doorbell and mirrors must be pinned host memory (%s)",
                            hipGetErrorString(e));
        }
        q = d;
    }
    hipLaunchKernelGGL(k_manage_gather, dim3(nwg), dim3(MANAGE_THREADS), 0, stream, st->e2s, st->s2e, st->last,
                       st->freq, st->step, st->E, st->S, policy, ids, n_ids, w, slot_ids, miss, n_miss, host_miss,
                       n_host, stats, dev_host, reinterpret_cast<unsigned char*>(slot_store), (uint64_t)slab_bytes,
                       sync, seq, reinterpret_cast<moe_doorbell*>(dptr[0]), reinterpret_cast<int32_t*>(dptr[1]),
                       reinterpret_cast<int32_t*>(dptr[2]), reinterpret_cast<float*>(dptr[3]),
                       g_fused_spin_limit.load(std::memory_order_relaxed));
    return moe_check_launch("cache_manage_gather");
}

int64_t moe_fused_spin_limit(int64_t polls) {
    if (polls > (int64_t)UINT32_MAX) polls = UINT32_MAX;
    if (polls < 0) return g_fused_spin_limit.load();
    return g_fused_spin_limit.exchange((uint32_t)polls);
}

int cache_repick(const moe_cache_state* st, const int32_t* want, int32_t* miss, int32_t* n_miss, hipStream_t stream) {
    int rc = check_state(st, "cache_repick");
    if (rc) return rc;
    MOE_REQUIRE(want && miss && n_miss, MOE_E_ARG, "cache_repick: want, miss and n_miss must be non-NULL");
    if (st->S == 0) return moe_ok();
    hipLaunchKernelGGL(k_repick, dim3(1), dim3(MANAGE_THREADS), 0, stream, st->e2s, st->s2e, st->last, st->freq,
                       st->step, st->E, st->S, want, miss, n_miss);
    return moe_check_launch("cache_repick");
}

int cache_gather(const int32_t* miss, const int32_t* n_miss, int max_miss, const void* host_store, void* slot_store,
                 size_t slab_bytes, hipStream_t stream) {
    MOE_REQUIRE(miss && n_miss && host_store && slot_store && max_miss >= 0, MOE_E_ARG,
                "cache_gather: miss, n_miss, host_store and slot_store must be non-NULL");
    MOE_REQUIRE(slab_bytes > 0 && slab_bytes % 16 == 0 && moe_aligned16(host_store) && moe_aligned16(slot_store),
                MOE_E_ALIGN, "cache_gather: slab_bytes=%zu and both stores must be 16-byte multiples / aligned",
                slab_bytes);
    if (max_miss == 0) return moe_ok();
    // the device address of the pinned host store, looked up on every call
    void* dev = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dev, const_cast<void*>(host_store), 0);
    if (e != hipSuccess || !dev) {
        (void)hipGetLastError();  // do not leave the failed query as the runtime's pending error
        return moe_fail(MOE_E_ARG, "cache_gather: host_store is not pinned, device-visible host memory (%s)",
                        hipGetErrorString(e));
    }
    const uint64_t chunks = (uint64_t)max_miss * (slab_bytes / 16);
    uint64_t grid = (chunks + GATHER_THREADS * GATHER_UNROLL - 1) / (GATHER_THREADS * GATHER_UNROLL);
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)grid), dim3(GATHER_THREADS), 0, stream, miss, n_miss, max_miss,
                       reinterpret_cast<const unsigned char*>(dev), reinterpret_cast<unsigned char*>(slot_store),
                       (uint64_t)slab_bytes);
    return moe_check_launch("cache_gather");
}

}  // extern "C"

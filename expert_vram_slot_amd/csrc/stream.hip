// Streamed miss pass: index kernels for serving the picks of non-resident
// experts on the GPU from staging slots (large batches).
//
// sozai.app transcript "rtx-3060-run-35b-llamacpp", "Full Transcript": the
// concurrent CPU lane pays off only on small batches; on a big prompt batch
// the system switches it off and processes the batch the way it did before.
// Here that means the non-resident experts' weights go over the host link to
// the GPU, a chunk at a time, and the GPU FFN runs on them (the driver in
// step.cpp issues the gathers on the side stream so that the gather of one
// chunk overlaps the FFN of the previous one).  These kernels only build the
// index lists; the copies are cache_gather's and the arithmetic is
// moe_ffn_slots'.
#include "stream.hpp"

#include "common.hpp"

namespace {

__global__ void __launch_bounds__(256) k_stream_pos(const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ slot_ids, int P,
                                                    const int32_t* __restrict__ host_miss,
                                                    const int32_t* __restrict__ n_host, int32_t* __restrict__ pos) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int nh = *n_host;
    int r = -1;
    if (slot_ids[p] < 0) {
        const int e = ids[p];
        int lo = 0, hi = nh;  // host_miss is ascending: binary search
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (host_miss[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        if (lo < nh && host_miss[lo] == e) r = lo;
    }
    pos[p] = r;
}

__global__ void __launch_bounds__(256) k_stream_chunk(const int32_t* __restrict__ pos, int P,
                                                      const int32_t* __restrict__ host_miss,
                                                      const int32_t* __restrict__ n_host, int c0, int R, int base,
                                                      int32_t* __restrict__ cmiss, int32_t* __restrict__ n_cmiss,
                                                      int32_t* __restrict__ cslots) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < R) {
        const int nh = *n_host;
        const int i = threadIdx.x;
        if (c0 + i < nh) {
            cmiss[2 * i] = host_miss[c0 + i];
            cmiss[2 * i + 1] = base + i;
        }
        if (i == 0) *n_cmiss = max(0, min(R, nh - c0));
    }
    if (p >= P) return;
    const int q = pos[p] - c0;
    cslots[p] = (pos[p] >= 0 && q >= 0 && q < R) ? base + q : -1;
}

}  // namespace

int moe_stream_pos(const int32_t* ids, const int32_t* slot_ids, int P, const int32_t* host_miss,
                   const int32_t* n_host, int32_t* pos, hipStream_t st) {
    if (P <= 0) return moe_ok();
    hipLaunchKernelGGL(k_stream_pos, dim3((P + 255) / 256), dim3(256), 0, st, ids, slot_ids, P, host_miss, n_host,
                       pos);
    return moe_check_launch("moe_layer_step/stream_pos");
}

int moe_stream_chunk(const int32_t* pos, int P, const int32_t* host_miss, const int32_t* n_host, int c0, int R,
                     int base, int32_t* cmiss, int32_t* n_cmiss, int32_t* cslots, hipStream_t st) {
    MOE_REQUIRE(R >= 1 && R <= 256 && P >= 1, MOE_E_ARG, "moe_stream_chunk: R=%d P=%d out of range", R, P);
    hipLaunchKernelGGL(k_stream_chunk, dim3((P + 255) / 256), dim3(256), 0, st, pos, P, host_miss, n_host, c0, R,
                       base, cmiss, n_cmiss, cslots);
    return moe_check_launch("moe_layer_step/stream_chunk");
}

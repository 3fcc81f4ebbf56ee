// Shared device helpers and error plumbing of the gfx950 expert-slot library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_slot.h"

// ----------------------------------------------------------------- errors

// Record a one-line reason for the calling thread and return `code`.
int moe_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the reason (successful call).
int moe_ok();
// Check the last launch; returns MOE_OK or MOE_E_HIP with the kernel's name.
int moe_check_launch(const char* what);

#define MOE_REQUIRE(cond, code, ...)              \
    do {                                          \
        if (!(cond)) return moe_fail(code, __VA_ARGS__); \
    } while (0)

static inline bool moe_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side slab layout (shared by every entry point of the library).
int moe_layout(int w_type, int H, int I, moe_slab_layout_t* out);

// ------------------------------------------------------- device helpers

namespace moe {

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum of v over the 64 lanes of the wave (fixed butterfly order).
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, WAVE);
    return v;
}

// One butterfly level at lane stride S with LIVE values still live: pairs of
// lanes (l, l ^ S) swap halves, so the live count halves while each value
// gathers the partner's partial sum.  Recurses down to stride 1 at compile
// time (every index is a constant, so the values stay in registers).
template <int LIVE, int S, int N, typename T>
__device__ __forceinline__ void multi_sum_level(T (&v)[N], int lane, int& id) {
    if constexpr (S >= 1) {
        if constexpr (LIVE > 1) {
            constexpr int n = LIVE / 2;
            const bool up = (lane & S) != 0;
#pragma unroll
            for (int i = 0; i < n; ++i) {
                const T send = up ? v[i] : v[i + n];
                const T keep = up ? v[i + n] : v[i];
                v[i] = keep + __shfl_xor(send, S, WAVE);
            }
            if (up) id += n;
            multi_sum_level<n, S / 2>(v, lane, id);
        } else {
            v[0] += __shfl_xor(v[0], S, WAVE);
            multi_sum_level<1, S / 2>(v, lane, id);
        }
    }
}

// Reduce N per-lane values over the 64 lanes at once (N a power of two,
// N <= 64).  Each butterfly level halves the number of live values, so the
// whole reduction costs about N exchanges instead of 6N.  On return v[0] of
// lane l holds the full 64-lane sum of value index `idx`; lanes whose low
// log2(64/N) bits are zero are the designated holders of each index.
template <int N, typename T>
__device__ __forceinline__ T wave_multi_sum(T (&v)[N], int lane, int& idx) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    int id = 0;
    multi_sum_level<N, 32>(v, lane, id);
    idx = id;
    return v[0];
}

template <int N>
__device__ __forceinline__ bool multi_sum_holder(int lane) {
    return (lane & (64 / N - 1)) == 0;
}

// Exclusive prefix sum over a block of blockDim.x (multiple of 64) threads
// of one int per thread, in thread order.  `scratch` holds >= blockDim/64 + 1
// ints of LDS.  Returns the exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        int o = __shfl_up(incl, s, WAVE);
        if (lane >= s) incl += o;
    }
    if (lane == 63) scratch[wid] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int w = 0; w < nw; ++w) {
            int t = scratch[w];
            scratch[w] = acc;
            acc += t;
        }
        scratch[nw] = acc;
    }
    __syncthreads();
    int res = scratch[wid] + incl - v;
    *total = scratch[nw];
    __syncthreads();
    return res;
}

}  // namespace moe

// Router for the expert-slot MoE layer on gfx950: logits, graded selection
// bias, top-k and the selection-only softmax weights.
//
// "Nudge, don't cut" (oois.ee/pgo-sgb), section "The method in five lines":
// the bias table is max(cap, ln(b / b_edge)) per cold expert and 0 for the hot
// set; top-k is taken on logit + bias; the weights are the router's own
// softmax over the k picked experts, computed from the unbiased logits.
//
// Logits are accumulated in double and rounded once to fp32, so the picks do
// not depend on a summation order that fp32 would expose at near-ties.
#include <math.h>

#include "common.hpp"

namespace {

constexpr int ROUTE_THREADS = 256;           // 4 waves: split over the hidden dimension
constexpr int ROUTE_KSPLIT = ROUTE_THREADS / 64;
constexpr int ROUTE_EJ = 8;                  // experts per lane per chunk (chunk = 512 experts)
constexpr int ROUTE_ECHUNK = 64 * ROUTE_EJ;

template <int XD>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
    if constexpr (XD == MOE_X_F32) return reinterpret_cast<const float*>(p)[i];
    else return moe::bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// ---------------------------------------------------------------- bias table

__global__ void __launch_bounds__(1024) k_bias_table(const double* __restrict__ b, int E, int n_hot, float cap,
                                                     float* __restrict__ bias) {
    __shared__ double sb[MOE_MAX_E];
    __shared__ unsigned char hot[MOE_MAX_E];
    __shared__ int s_edge;
    for (int e = threadIdx.x; e < E; e += blockDim.x) sb[e] = b[e];
    if (threadIdx.x == 0) s_edge = 0;
    __syncthreads();
    // rank of e: experts strictly brighter, or equally bright with a lower id
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const double be = sb[e];
        int rank = 0;
        for (int o = 0; o < E; ++o) {
            const double bo = sb[o];
            rank += (bo > be) || (bo == be && o < e);
        }
        if (rank == n_hot - 1) s_edge = e;  // exactly one expert has this rank
        hot[e] = rank < n_hot;
    }
    __syncthreads();
    const double b_edge = sb[s_edge];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        if (hot[e]) {
            bias[e] = 0.0f;
            continue;
        }
        const double be = sb[e];
        const double v = (be > 0.0 && b_edge > 0.0) ? log(be / b_edge) : -INFINITY;
        bias[e] = (float)(v > (double)cap ? v : (double)cap);
    }
}

// ----------------------------------------------------------------- router

// One workgroup routes TB consecutive tokens.  Logits: the 4 waves split the
// hidden dimension, each lane owns experts lane + 64 j of a 512-expert chunk,
// fp64 partial sums are combined wave 0 + 1 + 2 + 3 in that order.  Top-k:
// one wave per token, k rounds of a wave arg-max on (score desc, id asc).
template <int XD, int TB>
__global__ void __launch_bounds__(ROUTE_THREADS) k_route(const void* __restrict__ x, const void* __restrict__ G,
                                                         const float* __restrict__ bias,
                                                         const int32_t* __restrict__ ids_in, int T, int H, int E,
                                                         int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                                         float* __restrict__ logits) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int xbytes = XD == MOE_X_F32 ? 4 : 2;
    // x tile, transposed [H][TB]; partial sums [TB][512] double; logits [TB][E] float
    unsigned char* xs = smem;
    double* part = reinterpret_cast<double*>(smem + (((size_t)H * TB * xbytes + 15) & ~(size_t)15));
    float* zl = reinterpret_cast<float*>(part + TB * ROUTE_ECHUNK);

    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

    for (int i = threadIdx.x; i < H * TB; i += ROUTE_THREADS) {
        const int h = i / TB, t = i % TB;
        if constexpr (XD == MOE_X_F32) {
            reinterpret_cast<float*>(xs)[i] = t < nt ? reinterpret_cast<const float*>(x)[(int64_t)(t0 + t) * H + h] : 0.f;
        } else {
            reinterpret_cast<uint16_t*>(xs)[i] =
                t < nt ? reinterpret_cast<const uint16_t*>(x)[(int64_t)(t0 + t) * H + h] : (uint16_t)0;
        }
    }
    __syncthreads();

    const int hper = (H + ROUTE_KSPLIT - 1) / ROUTE_KSPLIT;
    const int h0 = wv * hper, h1 = min(H, h0 + hper);
    for (int ec = 0; ec < E; ec += ROUTE_ECHUNK) {
        double acc[TB][ROUTE_EJ];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < ROUTE_EJ; ++j) acc[t][j] = 0.0;
        for (int h = h0; h < h1; ++h) {
            double xv[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                if constexpr (XD == MOE_X_F32) xv[t] = reinterpret_cast<const float*>(xs)[h * TB + t];
                else xv[t] = moe::bf16_to_f32(reinterpret_cast<const uint16_t*>(xs)[h * TB + t]);
            }
#pragma unroll
            for (int j = 0; j < ROUTE_EJ; ++j) {
                const int e = ec + lane + 64 * j;
                if (e < E) {
                    const double g = load_act<XD>(G, (int64_t)h * E + e);
#pragma unroll
                    for (int t = 0; t < TB; ++t) acc[t][j] = fma(xv[t], g, acc[t][j]);
                }
            }
        }
        // fixed-order combination of the 4 partial sums
        for (int ww = 0; ww < ROUTE_KSPLIT; ++ww) {
            if (wv == ww) {
#pragma unroll
                for (int t = 0; t < TB; ++t)
#pragma unroll
                    for (int j = 0; j < ROUTE_EJ; ++j) {
                        double* p = &part[t * ROUTE_ECHUNK + lane + 64 * j];
                        *p = ww == 0 ? acc[t][j] : *p + acc[t][j];
                    }
            }
            __syncthreads();
        }
        for (int i = threadIdx.x; i < TB * ROUTE_ECHUNK; i += ROUTE_THREADS) {
            const int t = i / ROUTE_ECHUNK, e = ec + i % ROUTE_ECHUNK;
            if (e < E) zl[t * E + e] = (float)part[i];
        }
        __syncthreads();
    }

    if (logits) {
        for (int i = threadIdx.x; i < nt * E; i += ROUTE_THREADS)
            logits[(int64_t)t0 * E + i] = zl[i];
    }

    // one wave per token
    for (int t = wv; t < nt; t += ROUTE_KSPLIT) {
        const float* z = zl + t * E;
        int32_t pick = -1;  // lane j < k ends up holding the j-th pick
        if (ids_in) {
            if (lane < k) pick = ids_in[(int64_t)(t0 + t) * k + lane];
        } else {
            // scores of this lane's experts; taken experts become -inf (never re-picked)
            uint64_t taken = 0;  // bit j: expert lane + 64 j already picked (E <= 4096)
            for (int r = 0; r < k; ++r) {
                float best = -INFINITY;
                int be = 0x7FFFFFFF;
                for (int j = 0; lane + 64 * j < E; ++j) {
                    if (taken >> j & 1) continue;
                    const int e = lane + 64 * j;
                    float s = z[e];
                    if (bias) s = s + bias[e];
                    if (s > best || (s == best && e < be)) { best = s; be = e; }
                }
#pragma unroll
                for (int sft = 32; sft >= 1; sft >>= 1) {
                    const float ob = __shfl_xor(best, sft, 64);
                    const int oe = __shfl_xor(be, sft, 64);
                    if (ob > best || (ob == best && oe < be)) { best = ob; be = oe; }
                }
                if (lane == (be & 63)) taken |= 1ull << (be >> 6);
                if (lane == r) pick = be;
            }
            if (lane < k) ids[(int64_t)(t0 + t) * k + lane] = pick;
        }
        // softmax of the raw logits over the picks, in double
        // externally given picks are trusted to lie in [0, E); clamp only to keep the read in bounds
        double zj = lane < k ? (double)z[min(max(pick, 0), E - 1)] : -INFINITY;
        double m = zj;
#pragma unroll
        for (int sft = 32; sft >= 1; sft >>= 1) m = fmax(m, __shfl_xor(m, sft, 64));
        const double ej = lane < k ? exp(zj - m) : 0.0;
        const double sum = moe::wave_sum(ej);
        if (lane < k) w[(int64_t)(t0 + t) * k + lane] = (float)(ej / sum);
    }
}

template <int XD, int TB>
int launch_route(const void* x, const void* G, const float* bias, const int32_t* ids_in, int T, int H, int E, int k,
                 int32_t* ids, float* w, float* logits, hipStream_t s) {
    const int xbytes = XD == MOE_X_F32 ? 4 : 2;
    const size_t lds = (((size_t)H * TB * xbytes + 15) & ~(size_t)15) + sizeof(double) * TB * ROUTE_ECHUNK +
                       sizeof(float) * TB * E;
    if (lds > 160 * 1024) return moe_fail(MOE_E_SHAPE, "moe_route: H=%d E=%d need %zu B of LDS", H, E, lds);
    const int grid = (T + TB - 1) / TB;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_route<XD, TB>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_HIP, "moe_route: LDS attribute: %s", hipGetErrorString(e));
        }
    }
    hipLaunchKernelGGL((k_route<XD, TB>), dim3(grid), dim3(ROUTE_THREADS), lds, s, x, G, bias, ids_in, T, H, E, k,
                       ids, w, logits);
    return moe_check_launch("moe_route");
}

template <int XD>
int route_dispatch(const void* x, const void* G, const float* bias, const int32_t* ids_in, int T, int H, int E, int k,
                   int32_t* ids, float* w, float* logits, hipStream_t s) {
    const int xbytes = XD == MOE_X_F32 ? 4 : 2;
    // small batches: one token per workgroup (more workgroups, lower latency);
    // large batches: several tokens share each read of G
    int tb = T <= 256 ? 1 : 8;
    while (tb > 1 && ((size_t)H * tb * xbytes > 64 * 1024 || (size_t)E * tb * 4 > 32 * 1024)) tb >>= 1;
    switch (tb) {
        case 8: return launch_route<XD, 8>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, s);
        case 4: return launch_route<XD, 4>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, s);
        case 2: return launch_route<XD, 2>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, s);
        default: return launch_route<XD, 1>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, s);
    }
}

}  // namespace

extern "C" {

int moe_bias_table(const double* b, int E, int n_hot, float cap, float* bias, hipStream_t stream) {
    MOE_REQUIRE(b && bias, MOE_E_ARG, "moe_bias_table: b and bias must be non-NULL");
    MOE_REQUIRE(E >= 1 && n_hot >= 1, MOE_E_ARG, "moe_bias_table: E=%d and n_hot=%d must be >= 1", E, n_hot);
    MOE_REQUIRE(E <= MOE_MAX_E, MOE_E_SHAPE, "moe_bias_table: E=%d exceeds %d", E, MOE_MAX_E);
    MOE_REQUIRE(!(cap > 0.0f) && cap == cap, MOE_E_ARG, "moe_bias_table: cap=%g must be <= 0", (double)cap);
    if (n_hot > E) n_hot = E;
    hipLaunchKernelGGL(k_bias_table, dim3(1), dim3(1024), 0, stream, b, E, n_hot, cap, bias);
    return moe_check_launch("moe_bias_table");
}

int moe_route(const void* x, int x_dtype, const void* G, const float* bias, const int32_t* ids_in, int T, int H,
              int E, int k, int32_t* ids, float* w, float* logits, hipStream_t stream) {
    MOE_REQUIRE(x && G && w, MOE_E_ARG, "moe_route: x, G and w must be non-NULL");
    MOE_REQUIRE(ids_in || ids, MOE_E_ARG, "moe_route: ids must be non-NULL when ids_in is NULL");
    MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1, MOE_E_ARG, "moe_route: T=%d H=%d E=%d k=%d out of range", T, H,
                E, k);
    MOE_REQUIRE(k <= E && k <= MOE_MAX_K && E <= MOE_MAX_E, MOE_E_SHAPE,
                "moe_route: need k=%d <= E=%d, k <= %d, E <= %d", k, E, MOE_MAX_K, MOE_MAX_E);
    if (T == 0) return moe_ok();
    if (x_dtype == MOE_X_F32) return route_dispatch<MOE_X_F32>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, stream);
    if (x_dtype == MOE_X_BF16) return route_dispatch<MOE_X_BF16>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, stream);
    return moe_fail(MOE_E_DTYPE, "moe_route: unknown activation format %d", x_dtype);
}

}  // extern "C"

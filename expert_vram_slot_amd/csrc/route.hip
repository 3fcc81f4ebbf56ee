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

constexpr int ROUTE_THREADS = 256;  // 4 waves
constexpr int ROUTE_KSPLIT = ROUTE_THREADS / 64;

template <int XD>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
    if constexpr (XD == MOE_X_F32) return reinterpret_cast<const float*>(p)[i];
    else return moe::bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// ---------------------------------------------------------------- bias table

// FLAT: every cold expert gets `cap` itself (flat bias; -inf is the hard mask)
template <bool FLAT>
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
        if (FLAT) {
            bias[e] = cap;
            continue;
        }
        const double be = sb[e];
        const double v = (be > 0.0 && b_edge > 0.0) ? log(be / b_edge) : -INFINITY;
        bias[e] = (float)(v > (double)cap ? v : (double)cap);
    }
}

// Live-cache affinity: base (or 0) plus lambda for every expert with a slot.
__global__ void k_bias_affinity(const int32_t* __restrict__ e2s, const float* __restrict__ base, int E, float lambda,
                                float* __restrict__ bias) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    float v = base ? base[e] : 0.0f;
    if (e2s[e] >= 0) v = v + lambda;
    bias[e] = v;
}

// ----------------------------------------------------------------- router

using v4u = uint32_t __attribute__((ext_vector_type(4)));

// router rows (experts) per wave per pass: fewer when several tokens share a pass
template <int TB>
constexpr int route_rows() { return TB >= 4 ? 8 : 16; }

// Widen one 16-byte granule of the gate row to doubles (exact).
template <int XD>
__device__ __forceinline__ void widen(const v4u& g, double (&d)[XD == MOE_X_F32 ? 4 : 8]) {
    if constexpr (XD == MOE_X_F32) {
        d[0] = __uint_as_float(g.x);
        d[1] = __uint_as_float(g.y);
        d[2] = __uint_as_float(g.z);
        d[3] = __uint_as_float(g.w);
    } else {
        const uint32_t u[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = moe::bf16_lo(u[i]);
            d[2 * i + 1] = moe::bf16_hi(u[i]);
        }
    }
}

// Order-preserving code of a selection score: larger score, larger code;
// -0 and +0 share one code (they compare equal); every code is >= 1, and a
// NaN gets 1 (it never beats a number).  0 marks "absent or taken".
__device__ __forceinline__ uint32_t score_code(float f) {
    if (f != f) return 1u;
    if (f == 0.0f) return 0x80000000u;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    return __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(v), lane));
}

// Maximum of v over the 64 lanes of a wave (every lane active), the same on
// every lane: within each row of 16 lanes by DPP rotations by 8 and 4 and
// swaps within quads, then the four row maxima read out by lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o = dpp_u64<0x128>(v);  // row_ror:8
    v = o > v ? o : v;
    o = dpp_u64<0x124>(v);  // row_ror:4
    v = o > v ? o : v;
    o = dpp_u64<0x4E>(v);  // quad_perm [2,3,0,1]
    v = o > v ? o : v;
    o = dpp_u64<0xB1>(v);  // quad_perm [1,0,3,2]
    v = o > v ? o : v;
    uint64_t m = readlane_u64(v, 0);
    o = readlane_u64(v, 16);
    m = o > m ? o : m;
    o = readlane_u64(v, 32);
    m = o > m ? o : m;
    o = readlane_u64(v, 48);
    return o > m ? o : m;
}

// Top-k of one token's selection scores fl32(z[e] + bias[e]) on (score desc,
// id asc) by one wave, then the softmax over the picks, in double, of the
// raw logits z (selection only) or, with `damped`, of the biased scores;
// lane j < k ends up holding the j-th pick.  Lane l keeps the
// codes of experts l, l + 64, ... in registers (JM >= ceil(E / 64) of them),
// read once; each of the k rounds takes the lane's best code (the lowest
// expert on equal codes), a wave maximum of (code, ~expert), and clears the
// winner's code.  z and bias may be global or LDS.  Given picks (ids_in) are
// trusted to lie in [0, E) and clamped only to keep the read in bounds.
template <int JM>
__device__ __forceinline__ void topk_softmax(const float* z, const float* __restrict__ bias,
                                             const int32_t* __restrict__ ids_in, int E, int k, int t,
                                             int32_t* __restrict__ ids, float* __restrict__ w, bool damped) {
    const int lane = threadIdx.x & 63;
    int32_t pick = -1;
    if (ids_in) {
        if (lane < k) pick = ids_in[(int64_t)t * k + lane];
    } else {
        // all loads issued before any is used (addresses clamped, not branched)
        float sc[JM];
#pragma unroll
        for (int j = 0; j < JM; ++j) sc[j] = z[min(lane + 64 * j, E - 1)];
        if (bias) {
            float bv[JM];
#pragma unroll
            for (int j = 0; j < JM; ++j) bv[j] = bias[min(lane + 64 * j, E - 1)];
#pragma unroll
            for (int j = 0; j < JM; ++j) sc[j] = sc[j] + bv[j];
        }
        uint32_t code[JM];
#pragma unroll
        for (int j = 0; j < JM; ++j) code[j] = lane + 64 * j < E ? score_code(sc[j]) : 0u;
        for (int r = 0; r < k; ++r) {
            uint32_t bc = 0u;
            int bj = 0;
#pragma unroll
            for (int j = 0; j < JM; ++j) {
                if (code[j] > bc) {
                    bc = code[j];
                    bj = j;
                }
            }
            const uint64_t mine = bc ? ((uint64_t)bc << 32) | (uint32_t)~(uint32_t)(lane + 64 * bj) : 0ull;
            const int e = (int)~(uint32_t)wave_max_u64(mine);
            if (lane == (e & 63)) {
#pragma unroll
                for (int j = 0; j < JM; ++j)
                    if (j == (e >> 6)) code[j] = 0u;
            }
            if (lane == r) pick = e;
        }
        if (lane < k) ids[(int64_t)t * k + lane] = pick;
    }
    // the softmax input: the raw logit, or with `damped` the biased score
    double zj = -INFINITY;
    if (lane < k) {
        const int pe = min(max(pick, 0), E - 1);
        float v = z[pe];
        if (damped && bias) v = v + bias[pe];
        zj = (double)v;
    }
    double m = -INFINITY;
    for (int j = 0; j < k; ++j) m = fmax(m, readlane_f64(zj, j));
    const double ej = lane < k ? exp(zj - m) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += readlane_f64(ej, j);
    if (lane < k) w[(int64_t)t * k + lane] = (float)(ej / sum);
}

// topk_softmax with the register count picked for E at run time
__device__ __forceinline__ void topk_softmax_any(const float* z, const float* __restrict__ bias,
                                                 const int32_t* __restrict__ ids_in, int E, int k, int t,
                                                 int32_t* __restrict__ ids, float* __restrict__ w, bool damped) {
    if (E <= 256) topk_softmax<4>(z, bias, ids_in, E, k, t, ids, w, damped);
    else if (E <= 1024) topk_softmax<16>(z, bias, ids_in, E, k, t, ids, w, damped);
    else topk_softmax<64>(z, bias, ids_in, E, k, t, ids, w, damped);
}

// One workgroup routes TB consecutive tokens.  Logits: G is [E][H]; each wave
// takes ROUTE_RW expert rows per pass, its lanes read consecutive 16-byte
// granules of a row, the tokens sit in LDS widened to double, partial sums
// are fp64 FMAs reduced across the wave in one multi-value butterfly (fixed
// order), then rounded once to fp32.  Top-k: one wave per token, k rounds of
// a wave arg-max on (score desc, id asc).  Softmax of the raw logits over the
// picks in double.
template <int XD, int TB>
__global__ void __launch_bounds__(ROUTE_THREADS) k_route(const void* __restrict__ x, const void* __restrict__ G,
                                                         const float* __restrict__ bias,
                                                         const int32_t* __restrict__ ids_in, int T, int H, int E,
                                                         int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                                         float* __restrict__ logits, int damped) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int EPG = XD == MOE_X_F32 ? 4 : 8;  // elements per 16-byte granule
    constexpr int ROUTE_RW = route_rows<TB>();
    constexpr int V = ROUTE_RW * TB;
    double* xd = reinterpret_cast<double*>(smem);               // [TB][H]
    float* zl = reinterpret_cast<float*>(xd + (size_t)TB * H);  // [TB][E]

    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

    for (int i = threadIdx.x; i < TB * H; i += ROUTE_THREADS) {
        const int t = i / H, h = i % H;
        xd[i] = t < nt ? (double)load_act<XD>(x, (int64_t)(t0 + t) * H + h) : 0.0;
    }
    __syncthreads();

    const int KG = H / EPG;
    const int nfull = KG >> 6, tail = KG & 63;
    const size_t row_bytes = (size_t)KG * 16;
    const unsigned char* Gb = reinterpret_cast<const unsigned char*>(G);
    for (int e0 = 0; e0 < E; e0 += ROUTE_KSPLIT * ROUTE_RW) {
        const int ebase = e0 + wv * ROUTE_RW;
        double acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0;
        for (int c = 0; c <= nfull; ++c) {
            if (c == nfull && tail == 0) break;
            const bool last = c == nfull;
            const int g = (c << 6) + (last ? min(lane, tail - 1) : lane);
            const bool on = !last || lane < tail;
            v4u gr[ROUTE_RW];
#pragma unroll
            for (int r = 0; r < ROUTE_RW; ++r) {
                const int e = min(ebase + r, E - 1);  // rows past E are computed on a valid row and dropped
                gr[r] = *reinterpret_cast<const v4u*>(Gb + e * row_bytes + (size_t)g * 16);
                if (!on) gr[r] = v4u{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                double xv[EPG];
#pragma unroll
                for (int i = 0; i < EPG; ++i) xv[i] = xd[(size_t)t * H + (size_t)g * EPG + i];
#pragma unroll
                for (int r = 0; r < ROUTE_RW; ++r) {
                    double gd[EPG];
                    widen<XD>(gr[r], gd);
                    double a = acc[r * TB + t];
#pragma unroll
                    for (int i = 0; i < EPG; ++i) a = fma(xv[i], gd[i], a);
                    acc[r * TB + t] = a;
                }
            }
        }
        int idx;
        const double v = moe::wave_multi_sum<V>(acc, lane, idx);
        if (moe::multi_sum_holder<V>(lane)) {
            const int r = idx / TB, t = idx % TB;
            const int e = ebase + r;
            if (e < E && t < nt) zl[t * E + e] = (float)v;
        }
    }
    __syncthreads();

    if (logits) {
        for (int i = threadIdx.x; i < nt * E; i += ROUTE_THREADS) logits[(int64_t)t0 * E + i] = zl[i];
    }

    // one wave per token
    for (int t = wv; t < nt; t += ROUTE_KSPLIT) topk_softmax_any(zl + t * E, bias, ids_in, E, k, t0 + t, ids, w, damped != 0);
}

// ----------------------------------------------------- two-kernel router

// Logits of TB tokens against one block of 4 * RW expert rows per
// workgroup, written to z[T][E]: the tokens sit in LDS in their own format
// and are widened to double where used; each wave takes RW rows, its lanes
// read consecutive 16-byte granules of each row, fp64 FMAs, one multi-value
// butterfly per wave, rounded once to fp32.  Many workgroups share G, so
// small batches are not limited by one workgroup's read of the whole gate.
template <int XD, int TB, int RW>
__global__ void __launch_bounds__(ROUTE_THREADS) k_logits(const void* __restrict__ x, const void* __restrict__ G,
                                                          int T, int H, int E, float* __restrict__ z) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int EPG = XD == MOE_X_F32 ? 4 : 8;
    constexpr int XB = XD == MOE_X_F32 ? 4 : 2;
    constexpr int V = RW * TB;
    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ebase = blockIdx.y * (ROUTE_KSPLIT * RW) + wv * RW;
    const int KG = H / EPG;
    const size_t row_bytes = (size_t)KG * 16;
    // tokens to LDS, 16 bytes per thread and step; rows past T are zero
    const unsigned char* xb = reinterpret_cast<const unsigned char*>(x);
    for (int i = threadIdx.x; i < TB * KG; i += ROUTE_THREADS) {
        const int t = i / KG, g = i % KG;
        v4u v = v4u{0u, 0u, 0u, 0u};
        if (t < nt) v = *reinterpret_cast<const v4u*>(xb + (size_t)(t0 + t) * row_bytes + (size_t)g * 16);
        *reinterpret_cast<v4u*>(smem + (size_t)t * row_bytes + (size_t)g * 16) = v;
    }
    __syncthreads();
    if (ebase >= E) return;
    const unsigned char* Gb = reinterpret_cast<const unsigned char*>(G);
    double acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0;
    // U passes of 64 granules per chunk: every load of a chunk is issued
    // before the first is used; granules past the row are read clamped and
    // enter as zeros (adding +0 changes no sum); the sums still run pass by
    // pass, lane by lane
    constexpr int U = 4;
    for (int g0 = 0; g0 < KG; g0 += 64 * U) {
        v4u gr[U][RW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + 64 * u + lane;
            const int gc = g < KG ? g : KG - 1;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int e = min(ebase + r, E - 1);  // rows past E are computed on a valid row and dropped
                gr[u][r] = *reinterpret_cast<const v4u*>(Gb + e * row_bytes + (size_t)gc * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + 64 * u + lane;
            const bool on = g < KG;
            const int gc = on ? g : KG - 1;
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                double xv[EPG];
                widen<XD>(*reinterpret_cast<const v4u*>(smem + (size_t)t * row_bytes + (size_t)gc * 16), xv);
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    double gd[EPG];
                    widen<XD>(on ? gr[u][r] : v4u{0u, 0u, 0u, 0u}, gd);
                    double a = acc[r * TB + t];
#pragma unroll
                    for (int i = 0; i < EPG; ++i) a = fma(xv[i], gd[i], a);
                    acc[r * TB + t] = a;
                }
            }
        }
    }
    int idx;
    const double v = moe::wave_multi_sum<V>(acc, lane, idx);
    if (moe::multi_sum_holder<V>(lane)) {
        const int r = idx / TB, t = idx % TB;
        const int e = ebase + r;
        if (e < E && t < nt) z[(int64_t)(t0 + t) * E + e] = (float)v;
    }
    (void)XB;
}

// Logits of large bf16 batches on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64): z[t][e] = sum_h x[t][h] G[e][h], the bf16 values
// widened exactly to fp64, fp64 sums, rounded once to fp32 (the same
// precision as k_logits, the terms summed in another order).  A workgroup
// takes 16 tokens x 32 experts: wave w the experts 16 (w % 2).. against half
// of h (w / 2), the two halves added in LDS at the end.  Per 32 inputs of h,
// lane (m, q) (m = lane % 16, q = lane / 16) loads 8 consecutive values of
// token row m and of expert row m at offset 8q; multiply s (0..7) takes value
// s of each, so the four lanes of a row cover the 32 inputs once.  Two
// accumulators (even and odd multiplies) keep two chains in flight, and the
// loads run LM_D blocks of 32 inputs ahead.  Rows past T or E are read
// clamped and not stored.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int LM_WT = 16;  // tokens and experts of a wave's tile
constexpr int LM_D = 4;    // blocks of 32 inputs in flight per wave
__global__ void __launch_bounds__(ROUTE_THREADS) k_logits_mfma(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ G, int T, int H, int E,
                                                              float* __restrict__ z) {
    __shared__ f64x4 part[2][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int et = wv & 1, kh = wv >> 1;  // expert tile, half of h
    const int t0 = blockIdx.x * LM_WT, e0 = blockIdx.y * (2 * LM_WT) + et * LM_WT;
    const int m = lane & 15, q = lane >> 4;
    const int nb = H / 32, nh = (nb + 1) / 2;             // blocks in all, in the first half
    const int b0 = kh ? nh : 0, b1 = kh ? nb : nh;       // this wave's blocks
    const uint16_t* xr = x + (size_t)min(t0 + m, T - 1) * H + 8 * q;
    const uint16_t* gr = G + (size_t)min(e0 + m, E - 1) * H + 8 * q;
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
    if (e0 < E && b0 < b1) {  // uniform over the wave
        v4u a[LM_D], b[LM_D];
#pragma unroll
        for (int d = 0; d < LM_D; ++d) {  // blocks past this wave's last are read clamped (unused)
            const size_t k = (size_t)min(b0 + d, b1 - 1) * 32;
            a[d] = *reinterpret_cast<const v4u*>(xr + k);
            b[d] = *reinterpret_cast<const v4u*>(gr + k);
        }
        for (int kb = b0; kb < b1; kb += LM_D) {
#pragma unroll
            for (int d = 0; d < LM_D; ++d) {
                double ad[8], bd[8];
                widen<MOE_X_BF16>(a[d], ad);
                widen<MOE_X_BF16>(b[d], bd);
                const size_t k = (size_t)min(kb + d + LM_D, b1 - 1) * 32;
                a[d] = *reinterpret_cast<const v4u*>(xr + k);
                b[d] = *reinterpret_cast<const v4u*>(gr + k);
                if (kb + d < b1) {
#pragma unroll
                    for (int s2 = 0; s2 < 8; s2 += 2) {
                        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(ad[s2], bd[s2], acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(ad[s2 + 1], bd[s2 + 1], acc1, 0, 0, 0);
                    }
                }
            }
        }
    }
    const f64x4 acc = acc0 + acc1;
    if (kh) part[et][lane] = acc;
    __syncthreads();
    if (kh || e0 >= E) return;
    const f64x4 sum = acc + part[et][lane];
    // element i of lane (m, q): token t0 + q + 4i, expert e0 + m
    const int e = e0 + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + q + 4 * i;
        if (t < T && e < E) z[(int64_t)t * E + e] = (float)sum[i];
    }
}

// Top-k and weights from z[T][E], one wave per token, the token's scores
// read straight into registers.
template <int JM>
__global__ void __launch_bounds__(ROUTE_THREADS) k_topk(const float* __restrict__ z, const float* __restrict__ bias,
                                                        const int32_t* __restrict__ ids_in, int T, int E, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ w, int damped) {
    const int t = blockIdx.x * ROUTE_KSPLIT + (int)(threadIdx.x >> 6);
    if (t >= T) return;
    topk_softmax<JM>(z + (int64_t)t * E, bias, ids_in, E, k, t, ids, w, damped != 0);
}

template <int XD, int TB>
int launch_logits(const void* x, const void* G, int T, int H, int E, float* z, hipStream_t s) {
    constexpr int RW = 4;
    const size_t lds = (size_t)TB * H * (XD == MOE_X_F32 ? 4 : 2);
    const dim3 grid((T + TB - 1) / TB, (E + ROUTE_KSPLIT * RW - 1) / (ROUTE_KSPLIT * RW));
    hipLaunchKernelGGL((k_logits<XD, TB, RW>), grid, dim3(ROUTE_THREADS), lds, s, x, G, T, H, E, z);
    return moe_check_launch("moe_route/logits");
}

template <int XD>
int route_split(const void* x, const void* G, const float* bias, const int32_t* ids_in, int T, int H, int E, int k,
                int32_t* ids, float* w, float* logits, int damped, hipStream_t s) {
    // tokens per workgroup: more for larger batches (fewer reads of G), within 64 KiB of LDS
    const size_t xrow = (size_t)H * (XD == MOE_X_F32 ? 4 : 2);
    int tb = T >= 512 ? 8 : T >= 128 ? 4 : T >= 32 ? 2 : 1;
    while (tb > 1 && tb * xrow > 64 * 1024) tb >>= 1;
    if (xrow > 64 * 1024) return moe_fail(MOE_E_SHAPE, "moe_route: H=%d is too long for one token in LDS", H);
    int rc;
    // the fp64 matrix cores for large batches (the 288-expert layer's 2048
    // tokens: 215 -> 121 us for logits and top-k)
    if (XD == MOE_X_BF16 && T >= 512 && H % 32 == 0) {
        const dim3 grid((T + LM_WT - 1) / LM_WT, (E + 2 * LM_WT - 1) / (2 * LM_WT));
        hipLaunchKernelGGL(k_logits_mfma, grid, dim3(ROUTE_THREADS), 0, s, reinterpret_cast<const uint16_t*>(x),
                           reinterpret_cast<const uint16_t*>(G), T, H, E, logits);
        rc = moe_check_launch("moe_route/logits_mfma");
    } else switch (tb) {
        case 8: rc = launch_logits<XD, 8>(x, G, T, H, E, logits, s); break;
        case 4: rc = launch_logits<XD, 4>(x, G, T, H, E, logits, s); break;
        case 2: rc = launch_logits<XD, 2>(x, G, T, H, E, logits, s); break;
        default: rc = launch_logits<XD, 1>(x, G, T, H, E, logits, s); break;
    }
    if (rc) return rc;
    const dim3 grid((T + ROUTE_KSPLIT - 1) / ROUTE_KSPLIT);
    const int nj = (E + 63) / 64;
    if (nj <= 2) hipLaunchKernelGGL(k_topk<2>, grid, dim3(ROUTE_THREADS), 0, s, logits, bias, ids_in, T, E, k, ids, w, damped);
    else if (nj <= 4) hipLaunchKernelGGL(k_topk<4>, grid, dim3(ROUTE_THREADS), 0, s, logits, bias, ids_in, T, E, k, ids, w, damped);
    else if (nj <= 8) hipLaunchKernelGGL(k_topk<8>, grid, dim3(ROUTE_THREADS), 0, s, logits, bias, ids_in, T, E, k, ids, w, damped);
    else if (nj <= 16) hipLaunchKernelGGL(k_topk<16>, grid, dim3(ROUTE_THREADS), 0, s, logits, bias, ids_in, T, E, k, ids, w, damped);
    else hipLaunchKernelGGL(k_topk<64>, grid, dim3(ROUTE_THREADS), 0, s, logits, bias, ids_in, T, E, k, ids, w, damped);
    return moe_check_launch("moe_route/topk");
}

template <int XD, int TB>
int launch_route(const void* x, const void* G, const float* bias, const int32_t* ids_in, int T, int H, int E, int k,
                 int32_t* ids, float* w, float* logits, int damped, hipStream_t s) {
    const size_t lds = sizeof(double) * TB * H + sizeof(float) * TB * E;
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
                       ids, w, logits, damped);
    return moe_check_launch("moe_route");
}

template <int XD>
int route_dispatch(const void* x, const void* G, const float* bias, const int32_t* ids_in, int T, int H, int E, int k,
                   int32_t* ids, float* w, float* logits, int damped, hipStream_t s) {
    // with a logits buffer the logits and the top-k run as two kernels (many
    // workgroups share the gate); without one, one fused kernel per token block
    if (logits) return route_split<XD>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, s);
    // small batches: one token per workgroup (more workgroups, lower latency);
    // large batches: several tokens share each read of G
    int tb = T <= 64 ? 1 : 4;
    while (tb > 1 && sizeof(double) * tb * H + sizeof(float) * tb * E > 80 * 1024) tb >>= 1;
    switch (tb) {
        case 4: return launch_route<XD, 4>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, s);
        case 2: return launch_route<XD, 2>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, s);
        default: return launch_route<XD, 1>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, s);
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
    hipLaunchKernelGGL(k_bias_table<false>, dim3(1), dim3(1024), 0, stream, b, E, n_hot, cap, bias);
    return moe_check_launch("moe_bias_table");
}

int moe_bias_flat(const double* b, int E, int n_hot, float value, float* bias, hipStream_t stream) {
    MOE_REQUIRE(b && bias, MOE_E_ARG, "moe_bias_flat: b and bias must be non-NULL");
    MOE_REQUIRE(E >= 1 && n_hot >= 1, MOE_E_ARG, "moe_bias_flat: E=%d and n_hot=%d must be >= 1", E, n_hot);
    MOE_REQUIRE(E <= MOE_MAX_E, MOE_E_SHAPE, "moe_bias_flat: E=%d exceeds %d", E, MOE_MAX_E);
    MOE_REQUIRE(!(value > 0.0f) && value == value, MOE_E_ARG, "moe_bias_flat: value=%g must be <= 0", (double)value);
    if (n_hot > E) n_hot = E;
    hipLaunchKernelGGL(k_bias_table<true>, dim3(1), dim3(1024), 0, stream, b, E, n_hot, value, bias);
    return moe_check_launch("moe_bias_flat");
}

int moe_bias_affinity(const int32_t* e2s, const float* base, int E, float lambda, float* bias, hipStream_t stream) {
    MOE_REQUIRE(e2s && bias, MOE_E_ARG, "moe_bias_affinity: e2s and bias must be non-NULL");
    MOE_REQUIRE(E >= 1, MOE_E_ARG, "moe_bias_affinity: E=%d must be >= 1", E);
    MOE_REQUIRE(E <= MOE_MAX_E, MOE_E_SHAPE, "moe_bias_affinity: E=%d exceeds %d", E, MOE_MAX_E);
    MOE_REQUIRE(lambda - lambda == 0.0f, MOE_E_ARG, "moe_bias_affinity: lambda=%g must be finite", (double)lambda);
    hipLaunchKernelGGL(k_bias_affinity, dim3((E + 255) / 256), dim3(256), 0, stream, e2s, base, E, lambda, bias);
    return moe_check_launch("moe_bias_affinity");
}

int moe_route_ex(const void* x, int x_dtype, const void* G, const float* bias, const int32_t* ids_in, int T, int H,
                 int E, int k, int flags, int32_t* ids, float* w, float* logits, hipStream_t stream) {
    MOE_REQUIRE(x && G && w, MOE_E_ARG, "moe_route: x, G and w must be non-NULL");
    MOE_REQUIRE(ids_in || ids, MOE_E_ARG, "moe_route: ids must be non-NULL when ids_in is NULL");
    MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1, MOE_E_ARG, "moe_route: T=%d H=%d E=%d k=%d out of range", T, H,
                E, k);
    MOE_REQUIRE((flags & ~MOE_ROUTE_DAMPED) == 0, MOE_E_ARG, "moe_route: unknown flags 0x%x", flags);
    MOE_REQUIRE(k <= E && k <= MOE_MAX_K && E <= MOE_MAX_E, MOE_E_SHAPE,
                "moe_route: need k=%d <= E=%d, k <= %d, E <= %d", k, E, MOE_MAX_K, MOE_MAX_E);
    if (T == 0) return moe_ok();
    MOE_REQUIRE(moe_aligned16(x) && moe_aligned16(G), MOE_E_ALIGN, "moe_route: x and G must be 16-byte aligned");
    MOE_REQUIRE(H % (x_dtype == MOE_X_F32 ? 4 : 8) == 0, MOE_E_ALIGN,
                "moe_route: H=%d must fill whole 16-byte granules", H);
    const int damped = (flags & MOE_ROUTE_DAMPED) ? 1 : 0;
    if (x_dtype == MOE_X_F32)
        return route_dispatch<MOE_X_F32>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, stream);
    if (x_dtype == MOE_X_BF16)
        return route_dispatch<MOE_X_BF16>(x, G, bias, ids_in, T, H, E, k, ids, w, logits, damped, stream);
    return moe_fail(MOE_E_DTYPE, "moe_route: unknown activation format %d", x_dtype);
}

int moe_route(const void* x, int x_dtype, const void* G, const float* bias, const int32_t* ids_in, int T, int H,
              int E, int k, int32_t* ids, float* w, float* logits, hipStream_t stream) {
    return moe_route_ex(x, x_dtype, G, bias, ids_in, T, H, E, k, 0, ids, w, logits, stream);
}

}  // extern "C"

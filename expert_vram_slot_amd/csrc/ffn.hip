// Grouped SwiGLU expert FFN over resident slots (decode-sized token groups),
// with zero-return for picks whose expert is not resident.
//
// sozai.app transcript "rtx-3060-run-35b-llamacpp", "What the video covers" /
// "Full Transcript": the GPU expert step returns zeros for an expert that is
// not on the GPU, so a separate pass over the remaining experts can be added
// in.  Here a pick with slot -1 is simply never scheduled; the output row of a
// token with no resident pick is written as +0.0.
//
// Pipeline (all on the caller's stream, deterministic):
//   k_group      stable counting sort of the T*k picks by slot (one workgroup,
//                ballot-matched ranks, no atomics) -> per-slot pick lists and
//                the list of slots with work; above GROUP_MULTI_P picks the
//                same sort runs over 1024-pick chunks in two launches
//                (k_group_hist: per-chunk slot counts; k_group_place: offsets
//                and ranks, one workgroup per chunk); one-token batches of
//                the fp32, bf16 and 4-bit formats skip it (each workgroup of
//                the next two kernels takes one pick)
//   k_quant_rows (W8A8) int8 codes + scale per token
//   k_gu         gate and up rows of a slot against the slot's tokens, SwiGLU
//                epilogue -> h[pick][I]
//   k_quant_rows (W8A8) int8 codes + scale per pick of h
//   k_down       down rows against h -> part[pick][H] = w * o
//   k_reduce     y[t] = sum over resident picks in top-k order
//   (one token, fp32 / bf16 / 4-bit: k_gu with one pick per workgroup, then
//   k_down_tok, the down rows of all the token's picks and their sum)
//
// Weight streaming: each workgroup owns a tile of rows of one slot; the four
// waves split the rows, the 64 lanes of a wave read consecutive 16-byte
// granules of a row (coalesced 1 KiB per wave load), the slot's tokens are
// read from L2, and the per-lane partial sums of all rows and tokens are
// reduced across the wave in one multi-value butterfly.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "prefill.hpp"

// The workspace of moe_ffn_slots_noalloc: one array per device, in the code
// object, held until the process ends.  In host code `scratch` only names the
// array (a host-side stand-in, not a device address): its device address is
// looked up per device with hipGetSymbolAddress and kept in scratch_dev below.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

using v4u = uint32_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int FFN_THREADS = 256;
constexpr int NTMAX = 4;       // tokens of one slot handled per pass
constexpr int GROUP_THREADS = 1024;
constexpr bool X_PREFETCH = true;  // activation granules one chunk ahead (16-byte activation granules)
constexpr int GROUP_MULTI_P = 4096;  // larger batches sort with one workgroup per 1024 picks
// bf16 batches with at least this many picks take the MFMA grouped-GEMM path
// (128-expert 2048 x 768 layer, 64 slots: at 32 tokens 96 vs 102 us for the
// row-streaming kernels; at 16 tokens 82 vs 77, at 8 tokens 58 vs 55)
constexpr int PF_MIN_P = 256;
// and W8A8 batches from this many (int8 MFMA tiles; measured on the 128-expert, 2048 x 768 layer with 32
// slots: at 16 tokens a wash against the row-streaming kernels, 47 vs 49 us with every slot busy and 38 vs 33 us
// with half of them; from 32 tokens on the tiles win: 49 vs 63 us, 55 vs 99 at 64, 88 vs 341 at 256)
constexpr int PF_MIN_P_I8 = 256;

// ------------------------------------------------------------ formats

template <int F>
struct Fmt;
template <>
struct Fmt<MOE_W_F32> {
    static constexpr int REP = 1;  // row tiles per GEMV workgroup, taken one after the other
    static constexpr int RGU = 1;  // gate rows (and as many up rows) per wave
    static constexpr int RDN = 4;  // down rows per wave
    static constexpr int EPG = 4;       // weights per 16-byte granule
    static constexpr int ABYTES = 4;    // bytes per activation element in LDS
    using Acc = float;
};
template <>
struct Fmt<MOE_W_BF16> {
    static constexpr int REP = 1;  // row tiles per GEMV workgroup, taken one after the other
    static constexpr int RGU = 1;  // gate rows (and as many up rows) per wave
    static constexpr int RDN = 4;  // down rows per wave
    static constexpr int EPG = 8;
    static constexpr int ABYTES = 2;
    using Acc = float;
};
template <>
struct Fmt<MOE_W_W8A8> {
    static constexpr int REP = 1;  // row tiles per GEMV workgroup, taken one after the other
    // two gate rows (and two up rows) per wave: a 2 KiB row is two chunks of
    // 64 granules, so one row pair left each lane four loads in flight
    // (128-expert layer, 16 tokens, 32 busy slots: 51.8 -> 48.4 us); eight
    // down rows per wave on 32 lanes each (45.8 -> 45.0 us; 8 tokens 41.8 ->
    // 41.0 us, against four rows on 64 lanes)
    static constexpr int RGU = 2;  // gate rows (and as many up rows) per wave
    static constexpr int RDN = 8;  // down rows per wave
    static constexpr int EPG = 16;
    static constexpr int ABYTES = 1;
    using Acc = int;
};
template <>
struct Fmt<MOE_W_Q4B32> {
    // row tiles per GEMV workgroup, taken one after the other (two were better
    // with one gate/up row pair and four down rows per wave; with the counts
    // below one is: 32 tokens 62.2 -> 61.0 us, 1 token 13.3 -> 12.5 us)
    static constexpr int REP = 1;
    // 4-bit rows are short (a 2048-input row is one 64-granule chunk, a
    // 512-input down row 16 granules): two gate/up row pairs and eight down
    // rows per wave, the down rows on 16 lanes each, so every lane has loads
    // in flight (512-expert layer, 32 tokens: 94.6 -> 64.5 us; 1 token
    // unchanged)
    static constexpr int RGU = 2;  // gate rows (and as many up rows) per wave
    static constexpr int RDN = 8;  // down rows per wave
    static constexpr int EPG = 32;
    static constexpr int ABYTES = 2;
    using Acc = float;
};

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum of the 32 bf16 inputs of one 4-bit block (x0: inputs 0..7, x1: 8..15,
// x2: 16..23, x3: 24..31) in fp32, through the bf16 pair dot with (1, 1) in
// a fixed order: the one arithmetic of every block sum (made by the GEMV
// kernels themselves, or ahead of them by k_block_sums and the sort launch),
// so a token's bits do not depend on which made it.
__device__ __forceinline__ float block_sum_bf16(const v4u& x0, const v4u& x1, const v4u& x2, const v4u& x3) {
    constexpr uint32_t ONES = 0x3F803F80u;  // bf16 1.0 twice
    const uint32_t xv[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                             x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = dot2bf(xv[i], ONES, s);
    return s;
}

// 32 nibbles of one 4-bit block against its 32 bf16 inputs (x0 .. x3 as in
// block_sum_bf16).  Each code q becomes the bf16 value 128 + q (bits 0x4300 |
// q, exact), so a bf16 dot gives sum (q + 128) x; the block's sum of x
// (qxsum) removes the offset: sum (q - 8) x = sum (q + 128) x - 136 sum x.
// Input j of the block is the low nibble of byte j (j < 16) or the high
// nibble of byte j - 16.
__device__ __forceinline__ void granule_dot_q4(const v4u& w, const v4u& x0, const v4u& x1, const v4u& x2,
                                               const v4u& x3, float qscale, float qxsum, float& acc) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    const uint32_t xl[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t xh[8] = {x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = wv[i] & 0x0F0F0F0Fu;          // inputs 4i .. 4i+3
        const uint32_t hi = (wv[i] >> 4) & 0x0F0F0F0Fu;   // inputs 16+4i .. 16+4i+3
        d = dot2bf(__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u), xl[2 * i], d);
        d = dot2bf(__builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u), xl[2 * i + 1], d);
        d = dot2bf(__builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u), xh[2 * i], d);
        d = dot2bf(__builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u), xh[2 * i + 1], d);
    }
    acc = fmaf(qscale, fmaf(-136.0f, qxsum, d), acc);
}

// Accumulate one 16-byte weight granule against the matching activation
// granule `xa` (16 bytes for fp32/bf16/int8; 64 bytes of bf16 for 4-bit,
// with the block's input sum qxsum).
template <int F>
__device__ __forceinline__ void granule_dot(const v4u& w, const unsigned char* xa, float qscale, float qxsum,
                                            typename Fmt<F>::Acc& acc) {
    if constexpr (F == MOE_W_F32) {
        const float4 xv = *reinterpret_cast<const float4*>(xa);
        acc = fmaf(__uint_as_float(w.x), xv.x, acc);
        acc = fmaf(__uint_as_float(w.y), xv.y, acc);
        acc = fmaf(__uint_as_float(w.z), xv.z, acc);
        acc = fmaf(__uint_as_float(w.w), xv.w, acc);
    } else if constexpr (F == MOE_W_BF16) {
        const v4u xv = *reinterpret_cast<const v4u*>(xa);
        acc = dot2bf(w.x, xv.x, acc);
        acc = dot2bf(w.y, xv.y, acc);
        acc = dot2bf(w.z, xv.z, acc);
        acc = dot2bf(w.w, xv.w, acc);
    } else if constexpr (F == MOE_W_W8A8) {
        const v4u xv = *reinterpret_cast<const v4u*>(xa);
        acc = __builtin_amdgcn_sdot4((int)w.x, (int)xv.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.y, (int)xv.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.z, (int)xv.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.w, (int)xv.w, acc, false);
    } else {
        const v4u* xp = reinterpret_cast<const v4u*>(xa);
        granule_dot_q4(w, xp[0], xp[1], xp[2], xp[3], qscale, qxsum, acc);
    }
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// granule_dot for formats whose activation granule is 16 bytes (fp32, bf16,
// int8), with that granule already in registers.
template <int F>
__device__ __forceinline__ void granule_dot_reg(const v4u& w, const v4u& xv, typename Fmt<F>::Acc& acc) {
    static_assert(F != MOE_W_Q4B32, "4-bit activations span 64 bytes per granule");
    if constexpr (F == MOE_W_F32) {
        acc = fmaf(__uint_as_float(w.x), __uint_as_float(xv.x), acc);
        acc = fmaf(__uint_as_float(w.y), __uint_as_float(xv.y), acc);
        acc = fmaf(__uint_as_float(w.z), __uint_as_float(xv.z), acc);
        acc = fmaf(__uint_as_float(w.w), __uint_as_float(xv.w), acc);
    } else if constexpr (F == MOE_W_BF16) {
        acc = dot2bf(w.x, xv.x, acc);
        acc = dot2bf(w.y, xv.y, acc);
        acc = dot2bf(w.z, xv.z, acc);
        acc = dot2bf(w.w, xv.w, acc);
    } else {
        acc = __builtin_amdgcn_sdot4((int)w.x, (int)xv.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.y, (int)xv.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.z, (int)xv.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.w, (int)xv.w, acc, false);
    }
}


// ---------------------------------------------------------- workspace

struct WsLayout {
    size_t slot_off, pair_list, active, n_active, gcnt, pf_tiles, h, hq, hs, hmax, xq, xs, xbs, hbs, part, total;
};

WsLayout ws_layout(int T, int k, int S, int w_type, int H, int I) {
    WsLayout L{};
    const size_t P = (size_t)T * k;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t r = o;
        o = (o + bytes + 255) & ~(size_t)255;
        return r;
    };
    L.slot_off = take(4 * ((size_t)S + 1));
    L.pair_list = take(4 * (P ? P : 1));
    L.active = take(4 * (size_t)S);
    L.n_active = take(16);
    L.gcnt = take(P > (size_t)GROUP_MULTI_P ? 4 * ((P + GROUP_THREADS - 1) / GROUP_THREADS) * (size_t)S : 16);
    L.pf_tiles = take(moe_pf_tiles_bytes(T, k, S));
    const size_t hb = (w_type == MOE_W_BF16 || w_type == MOE_W_Q4B32) ? 2 : 4;
    L.h = take(hb * P * I);
    if (w_type == MOE_W_W8A8) {
        L.hq = take(P * I);
        L.hs = take(4 * P);
        L.hmax = take(4 * (P ? P : 1) * (size_t)((I + 63) / 64));
        L.xq = take((size_t)T * H);
        L.xs = take(4 * (size_t)T);
    }
    if (w_type == MOE_W_Q4B32) {
        L.xbs = take(4 * (size_t)T * (H / 32));
        L.hbs = take(4 * P * (I / 32));
    }
    L.part = take(4 * P * H);
    L.total = o;
    return L;
}

// ---------------------------------------------------------- grouping

// Rank of this lane's pick among the lanes of its wave holding the same slot
// (lane order), found with one ballot per bit of the slot id; *count gets the
// number of such lanes.  Lanes with valid == false take part in the ballots
// only.
__device__ __forceinline__ int wave_slot_rank(int s, bool valid, int nbits, int* count) {
    const uint64_t lt = (1ull << (threadIdx.x & 63)) - 1ull;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((s >> b) & 1);
        const uint64_t bm = __ballot(bit);
        mask &= bit ? bm : ~bm;
    }
    *count = __popcll(mask);
    return __popcll(mask & lt);
}

// Tiles of the grouped GEMM: ceil(cnt / mt) per slot, slots in ascending
// order.  Called by the whole workgroup (thread s holds slot s's pick count
// and offset; S <= blockDim.x); tiles == NULL writes nothing.
__device__ __forceinline__ void write_pf_tiles(int cnt, int off, int S, int mt, int* scan_lds, moe_pf_tile* tiles,
                                               int32_t* n_tiles) {
    if (!tiles) return;
    const int s = threadIdx.x;
    const int nc = (s < S) ? (cnt + mt - 1) / mt : 0;
    int tot;
    const int toff = moe::block_exclusive_scan(nc, scan_lds, &tot);
    for (int c = 0; c < nc; ++c) tiles[toff + c] = moe_pf_tile{off + c * mt, min(mt, cnt - c * mt), s, 0};
    if (threadIdx.x == 0) *n_tiles = tot;
}

// Activation preparation of a batch, by the workgroups 1.. of the sorting
// launch (workgroup 0 sorts): W8A8 codes and per-row scales of x, one
// workgroup per row (the arithmetic of k_quant_rows<true>), or the 32-input
// block sums of x for 4-bit weights, 1024 blocks per workgroup (that of
// k_block_sums).  Same bits as those kernels; one launch fewer.
enum { XPREP_NONE = 0, XPREP_I8 = 1, XPREP_BSUM = 2 };

__device__ void x_prep_wg(int kind, int wg, const uint16_t* __restrict__ x, int T, int H, int8_t* __restrict__ xq,
                          float* __restrict__ xs, float* __restrict__ xbs) {
    const int tid = threadIdx.x;
    if (kind == XPREP_I8) {
        __shared__ float red[GROUP_THREADS / 64];
        const uint16_t* row = x + (int64_t)wg * H;
        float m = 0.0f;
        for (int i = tid; i < H; i += GROUP_THREADS) m = fmaxf(m, fabsf(moe::bf16_to_f32(row[i])));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        float amax = 0.0f;
#pragma unroll
        for (int w = 0; w < GROUP_THREADS / 64; ++w) amax = fmaxf(amax, red[w]);
        const float sc = amax > 0.0f ? amax / 127.0f : 1.0f;
        for (int i = tid; i < H; i += GROUP_THREADS) {
            float c = rintf(moe::bf16_to_f32(row[i]) / sc);
            c = fminf(fmaxf(c, -127.0f), 127.0f);
            xq[(int64_t)wg * H + i] = (int8_t)c;
        }
        if (tid == 0) xs[wg] = sc;
    } else {
        const int nb = H / 32;
        const int64_t i = (int64_t)wg * GROUP_THREADS + tid;
        if (i >= (int64_t)T * nb) return;
        const v4u* p = reinterpret_cast<const v4u*>(x + (i / nb) * H + 32 * (i % nb));
        xbs[i] = block_sum_bf16(p[0], p[1], p[2], p[3]);
    }
}

// Workgroups the preparation of x takes in the sorting launch.
__host__ __device__ inline int x_prep_wgs(int kind, int T, int H) {
    return kind == XPREP_I8 ? T : kind == XPREP_BSUM ? (T * (H / 32) + GROUP_THREADS - 1) / GROUP_THREADS : 0;
}

// Stable counting sort of the P picks by slot.  Picks are taken 1024 at a
// time; inside a wave the picks with the same slot are found with one ballot
// per slot-id bit, their order is the lane order; per-wave counts are
// prefix-summed per slot across the 16 waves.  Pass 0 counts, pass 1 places.
__global__ void __launch_bounds__(GROUP_THREADS) k_group(const int32_t* __restrict__ slot_ids, int P, int S,
                                                         int32_t* __restrict__ slot_off, int32_t* __restrict__ pair_list,
                                                         int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                                         moe_pf_tile* __restrict__ pf_tiles,
                                                         int32_t* __restrict__ pf_n_tiles, int pf_mt, int xprep,
                                                         const uint16_t* __restrict__ x, int T, int H,
                                                         int8_t* __restrict__ xq, float* __restrict__ xs,
                                                         float* __restrict__ xbs) {
    if (blockIdx.x > 0) {  // workgroups 1..: x for the gate/up kernel
        x_prep_wg(xprep, blockIdx.x - 1, x, T, H, xq, xs, xbs);
        return;
    }
    __shared__ uint16_t wtab[GROUP_THREADS / 64][MOE_MAX_S];
    __shared__ int base[MOE_MAX_S];
    __shared__ int ctot[MOE_MAX_S];
    __shared__ int scan_lds[GROUP_THREADS / 64 + 1];
    const int tid = threadIdx.x, wid = tid >> 6;
    int nbits = 0;
    while ((1 << nbits) < S) ++nbits;

    if (P <= GROUP_THREADS) {
        // one chunk (every decode batch up to 1024 picks): counts, offsets
        // and places from one read of the slot ids
        for (int i = tid; i < (GROUP_THREADS / 64) * S; i += GROUP_THREADS) wtab[i / S][i % S] = 0;
        __syncthreads();
        const int p = tid;
        int s = p < P ? slot_ids[p] : -1;
        if (s >= S) s = -1;
        const bool valid = s >= 0;
        int cnt;
        const int rank = wave_slot_rank(s, valid, nbits, &cnt);
        if (valid && rank == 0) wtab[wid][s] = (uint16_t)cnt;
        __syncthreads();
        int tot_s = 0;
        if (tid < S) {
            for (int w = 0; w < GROUP_THREADS / 64; ++w) {
                const int c = wtab[w][tid];
                wtab[w][tid] = (uint16_t)tot_s;
                tot_s += c;
            }
        }
        int tot;
        const int off = moe::block_exclusive_scan(tot_s, scan_lds, &tot);
        if (tid < S) {
            slot_off[tid] = off;
            base[tid] = off;
        }
        if (tid == 0) slot_off[S] = tot;
        const int flag = (tid < S && tot_s > 0) ? 1 : 0;
        int na;
        const int apos = moe::block_exclusive_scan(flag, scan_lds, &na);
        if (flag) active[apos] = tid;
        if (tid == 0) *n_active = na;
        write_pf_tiles(tot_s, off, S, pf_mt, scan_lds, pf_tiles, pf_n_tiles);
        __syncthreads();
        if (valid) pair_list[base[s] + wtab[wid][s] + rank] = p;
        return;
    }
    for (int s = tid; s < S; s += GROUP_THREADS) base[s] = 0;
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
        for (int c0 = 0; c0 < P; c0 += GROUP_THREADS) {
            for (int i = tid; i < (GROUP_THREADS / 64) * S; i += GROUP_THREADS) wtab[i / S][i % S] = 0;
            __syncthreads();
            const int p = c0 + tid;
            int s = p < P ? slot_ids[p] : -1;
            if (s >= S) s = -1;
            const bool valid = s >= 0;
            int cnt;
            const int rank = wave_slot_rank(s, valid, nbits, &cnt);
            if (valid && rank == 0) wtab[wid][s] = (uint16_t)cnt;
            __syncthreads();
            for (int s2 = tid; s2 < S; s2 += GROUP_THREADS) {
                int acc = 0;
                for (int w = 0; w < GROUP_THREADS / 64; ++w) {
                    const int c = wtab[w][s2];
                    wtab[w][s2] = (uint16_t)acc;
                    acc += c;
                }
                ctot[s2] = acc;
            }
            __syncthreads();
            if (pass == 1 && valid) pair_list[base[s] + wtab[wid][s] + rank] = p;
            __syncthreads();
            for (int s2 = tid; s2 < S; s2 += GROUP_THREADS) base[s2] += ctot[s2];
            __syncthreads();
        }
        if (pass == 0) {
            // counts -> offsets; slots with work, ascending
            const int cnt = tid < S ? base[tid] : 0;
            int tot;
            const int off = moe::block_exclusive_scan(cnt, scan_lds, &tot);
            if (tid < S) {
                slot_off[tid] = off;
                base[tid] = off;
            }
            if (tid == 0) slot_off[S] = tot;
            const int flag = (tid < S && cnt > 0) ? 1 : 0;
            int na;
            const int apos = moe::block_exclusive_scan(flag, scan_lds, &na);
            if (flag) active[apos] = tid;
            if (tid == 0) *n_active = na;
            write_pf_tiles(cnt, off, S, pf_mt, scan_lds, pf_tiles, pf_n_tiles);
            __syncthreads();
        }
    }
}

// k_group's lists (slot_off, pair_list, active, n_active) for batches of at
// most 64 picks that need nothing else (fp32 and bf16 weights): one wave,
// one pick per lane; ranks within a slot from ballots (wave_slot_rank), the
// offsets by a wave prefix sum over the slots, 64 at a time.  (The
// 128-expert bf16 layer, 64 slots: 8 tokens 52.0 -> 50.2 us, 4 tokens
// 30.9 -> 29.2 us, back to back, against the 1024-thread sort.)
constexpr int GROUP_SMALL_P = 64;
__global__ void __launch_bounds__(64) k_group_small(const int32_t* __restrict__ slot_ids, int P, int S,
                                                    int32_t* __restrict__ slot_off, int32_t* __restrict__ pair_list,
                                                    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
    __shared__ int cnt[MOE_MAX_S];  // per slot: its pick count, then its first position
    const int lane = threadIdx.x;
    int nbits = 0;
    while ((1 << nbits) < S) ++nbits;
    int s = lane < P ? slot_ids[lane] : -1;
    if (s >= S) s = -1;
    const bool valid = s >= 0;
    for (int i = lane; i < S; i += 64) cnt[i] = 0;
    int c;
    const int rank = wave_slot_rank(s, valid, nbits, &c);
    __syncthreads();
    if (valid && rank == 0) cnt[s] = c;
    __syncthreads();
    const uint64_t lt = (1ull << lane) - 1ull;
    int carry = 0, acarry = 0;
    for (int base = 0; base < S; base += 64) {
        const int sl = base + lane;
        const int cv = sl < S ? cnt[sl] : 0;
        int incl = cv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        const uint64_t busy = __ballot(cv > 0);
        if (sl < S) {
            slot_off[sl] = carry + incl - cv;
            cnt[sl] = carry + incl - cv;
        }
        if (cv > 0) active[acarry + __popcll(busy & lt)] = sl;
        carry += __shfl(incl, 63, 64);
        acarry += __popcll(busy);
    }
    if (lane == 0) {
        slot_off[S] = carry;
        *n_active = acarry;
    }
    __syncthreads();
    if (valid) pair_list[cnt[s] + rank] = lane;
}

// Per-chunk slot counts: cnt[c][s] = picks of chunk c (1024 picks) with slot s.
__global__ void __launch_bounds__(GROUP_THREADS) k_group_hist(const int32_t* __restrict__ slot_ids, int P, int S,
                                                              int32_t* __restrict__ cnt) {
    __shared__ int c[MOE_MAX_S];
    const int tid = threadIdx.x;
    for (int s = tid; s < S; s += GROUP_THREADS) c[s] = 0;
    __syncthreads();
    const int p = blockIdx.x * GROUP_THREADS + tid;
    const int s = p < P ? slot_ids[p] : -1;
    if (s >= 0 && s < S) atomicAdd(&c[s], 1);  // LDS integer count: order-free
    __syncthreads();
    for (int s2 = tid; s2 < S; s2 += GROUP_THREADS) cnt[(size_t)blockIdx.x * S + s2] = c[s2];
}

// Places chunk c's picks: slot offsets from the per-chunk counts (prefix over
// slots of the totals, plus the counts of earlier chunks), then the stable
// rank inside the chunk as in k_group.  Chunk 0 also writes the slot offsets
// and the slots with work.  Same result as k_group.
__global__ void __launch_bounds__(GROUP_THREADS) k_group_place(const int32_t* __restrict__ slot_ids, int P, int S,
                                                               const int32_t* __restrict__ cnt, int nch,
                                                               int32_t* __restrict__ slot_off,
                                                               int32_t* __restrict__ pair_list,
                                                               int32_t* __restrict__ active,
                                                               int32_t* __restrict__ n_active,
                                                               moe_pf_tile* __restrict__ pf_tiles,
                                                               int32_t* __restrict__ pf_n_tiles, int pf_mt) {
    __shared__ uint16_t wtab[GROUP_THREADS / 64][MOE_MAX_S];
    __shared__ int base[MOE_MAX_S];
    __shared__ int scan_lds[GROUP_THREADS / 64 + 1];
    const int tid = threadIdx.x, wid = tid >> 6, c = blockIdx.x;
    int tot = 0, pre = 0;
    if (tid < S) {
        for (int cc = 0; cc < nch; ++cc) {
            const int v = cnt[(size_t)cc * S + tid];
            tot += v;
            pre += cc < c ? v : 0;
        }
    }
    int all;
    const int off = moe::block_exclusive_scan(tot, scan_lds, &all);
    if (tid < S) base[tid] = off + pre;
    if (c == 0) {
        if (tid < S) slot_off[tid] = off;
        if (tid == 0) slot_off[S] = all;
        const int flag = (tid < S && tot > 0) ? 1 : 0;
        int na;
        const int apos = moe::block_exclusive_scan(flag, scan_lds, &na);
        if (flag) active[apos] = tid;
        if (tid == 0) *n_active = na;
        write_pf_tiles(tot, off, S, pf_mt, scan_lds, pf_tiles, pf_n_tiles);
    }
    for (int i = tid; i < (GROUP_THREADS / 64) * S; i += GROUP_THREADS) wtab[i / S][i % S] = 0;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < S) ++nbits;
    const int p = c * GROUP_THREADS + tid;
    int s = p < P ? slot_ids[p] : -1;
    if (s >= S) s = -1;
    const bool valid = s >= 0;
    int count;
    const int rank = wave_slot_rank(s, valid, nbits, &count);
    if (valid && rank == 0) wtab[wid][s] = (uint16_t)count;
    __syncthreads();
    for (int s2 = tid; s2 < S; s2 += GROUP_THREADS) {
        int acc = 0;
        for (int w = 0; w < GROUP_THREADS / 64; ++w) {
            const int v = wtab[w][s2];
            wtab[w][s2] = (uint16_t)acc;
            acc += v;
        }
    }
    __syncthreads();
    if (valid) pair_list[base[s] + wtab[wid][s] + rank] = p;
}

// ------------------------------------------------------- W8A8 quantiser

// Per row: scale = absmax / 127 (1 if the row is all zero), code =
// clamp(rint(v / scale), -127, 127), in fp32.  Rows whose `valid` entry is
// negative (picks not resident) are skipped.  Rows of up to QR_VPT * 256
// values are read once, into registers, and the row's loads do not wait for
// its `valid` entry (the row is in bounds either way; a skipped row's values
// are dropped), so the kernel waits on one round of loads.
constexpr int QR_VPT = 8;
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) k_quant_rows(const void* __restrict__ src, int len,
                                                    const int32_t* __restrict__ valid, int8_t* __restrict__ q,
                                                    float* __restrict__ scale) {
    __shared__ float red[4];
    const int row = blockIdx.x;
    const bool ok = !valid || valid[row] >= 0;
    auto val = [&](int i) -> float {
        if constexpr (SRC_BF16) return moe::bf16_to_f32(reinterpret_cast<const uint16_t*>(src)[(int64_t)row * len + i]);
        else return reinterpret_cast<const float*>(src)[(int64_t)row * len + i];
    };
    const bool held = len <= QR_VPT * 256;
    float v[QR_VPT];
    float m = 0.0f;
    if (held) {
#pragma unroll
        for (int u = 0; u < QR_VPT; ++u) {
            const int i = threadIdx.x + 256 * u;
            v[u] = i < len ? val(i) : 0.0f;
            m = fmaxf(m, fabsf(v[u]));
        }
    } else {
        for (int i = threadIdx.x; i < len; i += 256) m = fmaxf(m, fabsf(val(i)));
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (!ok) return;  // the whole workgroup
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax > 0.0f ? amax / 127.0f : 1.0f;
    auto code = [&](float x) { return (int8_t)fminf(fmaxf(rintf(x / sc), -127.0f), 127.0f); };
    if (held) {
#pragma unroll
        for (int u = 0; u < QR_VPT; ++u) {
            const int i = threadIdx.x + 256 * u;
            if (i < len) q[(int64_t)row * len + i] = code(v[u]);
        }
    } else {
        for (int i = threadIdx.x; i < len; i += 256) q[(int64_t)row * len + i] = code(val(i));
    }
    if (threadIdx.x == 0) scale[row] = sc;
}

// ------------------------------------------------------ GEMV kernels

struct SlabView {
    const unsigned char* slots;
    size_t slab_bytes;
    int64_t w0, w1, s0, s1;  // weight and scale plane offsets used by the kernel
};

// Expert weights are streamed once per step: non-temporal loads keep them
// from displacing the small, reused data (tokens, pick lists) in the caches.
__device__ __forceinline__ v4u load_weights(const v4u* p) { return __builtin_nontemporal_load(p); }

// One wave's ROWS weight rows (row r at rowp[r]; 4-bit scale rows at scp[r]).
// Rows past the end are clamped to the last row (computed, then dropped) so
// every load stays in bounds.
template <int ROWS>
struct RowPtrs {
    const unsigned char* w[ROWS];
    const unsigned char* s[ROWS];
};

// Activations of one pass: up to NT rows of a row-major [rows][len] array
// (x for gate/up, h for down), read directly from global memory (they are
// small and shared by every tile of the slot, so they stay in L2).  4-bit
// weights also need the per-block sums of those rows (made by gemv_rows
// itself with INSUM, the one-token kernels).
struct ActRows {
    const unsigned char* base;  // row r at base + r * row_bytes
    size_t row_bytes;
    const float* bsum;          // [rows][len / 32] (4-bit only)
};

// Dot products of ROWS weight rows with NT activation rows over KG 16-byte
// granules.  The wave's lanes form 64 / LPR groups of LPR lanes; group s
// takes rows s, s + 64/LPR, ... and lane l of a group reads granules l,
// l + LPR, ... of its rows, so one wave load covers 64 / LPR rows (rows of
// fewer than 64 granules keep every lane busy).  Chunks of LPR granules go in
// groups of NCHG whose weight loads are all issued before the first is used;
// granules past the end read a clamped, in-bounds granule with zero weights.
// acc[i * NT + t] holds the lane's partial sum of its i-th row and token t.
template <int F, int ROWS, int NT, int NCHG, int LPR, bool INSUM = false>
__device__ __forceinline__ void gemv_rows(const RowPtrs<ROWS>& rp, const ActRows& ar, const int (&arow)[NT], int KG,
                                          int lane, typename Fmt<F>::Acc (&acc)[(ROWS * LPR / 64) * NT]) {
    constexpr int XG = Fmt<F>::EPG * Fmt<F>::ABYTES;  // activation bytes per weight granule
    constexpr int RPI = 64 / LPR;                      // rows per wave load
    constexpr int RL = ROWS / RPI;                     // rows per lane
    static_assert(ROWS % RPI == 0, "rows must fill the lane groups");
    const int sub = lane / LPR, gl = lane % LPR;
    // this lane's rows: sub + RPI * i (selected with constant indices only)
    const unsigned char* wrow[RL];
    const unsigned char* srow[RL];
#pragma unroll
    for (int i = 0; i < RL; ++i) {
        wrow[i] = rp.w[i * RPI];
        srow[i] = rp.s[i * RPI];
#pragma unroll
        for (int u = 1; u < RPI; ++u)
            if (sub == u) {
                wrow[i] = rp.w[i * RPI + u];
                srow[i] = rp.s[i * RPI + u];
            }
    }
    for (int g0 = 0; g0 < KG; g0 += LPR * NCHG) {
        v4u w[NCHG][RL];
        float qs[NCHG][RL];
        int gj[NCHG];
        bool on[NCHG];
#pragma unroll
        for (int j = 0; j < NCHG; ++j) {
            const int g = g0 + LPR * j + gl;
            on[j] = g < KG;
            gj[j] = on[j] ? g : KG - 1;
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                w[j][i] = load_weights(reinterpret_cast<const v4u*>(wrow[i] + (size_t)gj[j] * 16));
                qs[j][i] = 0.0f;
                if constexpr (F == MOE_W_Q4B32)
                    qs[j][i] = half_bits_to_f32(reinterpret_cast<const uint16_t*>(srow[i])[gj[j]]);
            }
        }
#pragma unroll
        for (int j = 0; j < NCHG; ++j) {
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                if (!on[j]) {
                    w[j][i] = v4u{0u, 0u, 0u, 0u};
                    qs[j][i] = 0.0f;
                }
            }
        }
        if constexpr (F == MOE_W_Q4B32 || !X_PREFETCH) {
#pragma unroll
            for (int j = 0; j < NCHG; ++j) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const unsigned char* xa = ar.base + (size_t)arow[t] * ar.row_bytes + (size_t)gj[j] * XG;
                    if constexpr (F == MOE_W_Q4B32 && INSUM) {
                        // one-token batches skip the launches that make the block sums: the
                        // block's inputs held once for all rows, their sum made here
                        const v4u* xp = reinterpret_cast<const v4u*>(xa);
                        const v4u x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
                        const float xsum = block_sum_bf16(x0, x1, x2, x3);
#pragma unroll
                        for (int i = 0; i < RL; ++i)
                            granule_dot_q4(w[j][i], x0, x1, x2, x3, qs[j][i], xsum, acc[i * NT + t]);
                    } else {
                        float xsum = 0.0f;
                        if constexpr (F == MOE_W_Q4B32) xsum = ar.bsum[(size_t)arow[t] * KG + gj[j]];
#pragma unroll
                        for (int i = 0; i < RL; ++i) granule_dot<F>(w[j][i], xa, qs[j][i], xsum, acc[i * NT + t]);
                    }
                }
            }
        } else {
            // activation granules of every token: chunk j + 1 in flight while chunk j is used
            v4u xr[2][NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                xr[0][t] = *reinterpret_cast<const v4u*>(ar.base + (size_t)arow[t] * ar.row_bytes + (size_t)gj[0] * 16);
#pragma unroll
            for (int j = 0; j < NCHG; ++j) {
                if (j + 1 < NCHG) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        xr[(j + 1) & 1][t] = *reinterpret_cast<const v4u*>(ar.base + (size_t)arow[t] * ar.row_bytes +
                                                                           (size_t)gj[j + 1] * 16);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int i = 0; i < RL; ++i) granule_dot_reg<F>(w[j][i], xr[j & 1][t], acc[i * NT + t]);
            }
        }
    }
}

// Chunk-group size for a row of KG granules read LPR at a time: the whole
// row when it has at most 4 chunks, else groups of 4.
__host__ __device__ constexpr int chunk_group(int KG, int LPR = 64) {
    return KG <= LPR ? 1 : KG <= 2 * LPR ? 2 : KG <= 3 * LPR ? 3 : 4;
}

// Lanes per row of the down projection.  Narrower lane groups keep every
// lane busy on short rows but give each lane fewer rows to share one
// activation read with.  fp32/bf16 rows take the widest group that divides
// them; int8 rows 32 lanes, with eight rows per wave (Fmt<MOE_W_W8A8>::RDN);
// 4-bit rows of up to 16 (32) granules 16 (32) lanes, with eight rows per
// wave (Fmt<MOE_W_Q4B32>::RDN).
__host__ __device__ constexpr int down_lpr(int KG, int w_type) {
    return w_type == MOE_W_Q4B32 ? (KG <= 16 ? 16 : KG <= 32 ? 32 : 64)
           : w_type == MOE_W_W8A8                                  ? 32
           : (KG % 64 == 0 || KG >= 128)                           ? 64
           : KG % 32 == 0                                                              ? 32
           : KG % 16 == 0                                                              ? 16
                                                                                       : 64;
}

#define MOE_NCHG_DISPATCH(KG, BODY)              \
    do {                                         \
        switch (chunk_group(KG)) {               \
            case 1: BODY(1); break;              \
            case 2: BODY(2); break;              \
            case 3: BODY(3); break;              \
            default: BODY(4); break;             \
        }                                        \
    } while (0)

#define MOE_DOWN_DISPATCH(KG, BODY)                                   \
    do {                                                              \
        const int lpr_ = down_lpr(KG, F);                             \
        const int g_ = chunk_group(KG, lpr_);                         \
        if (lpr_ == 16) {                                             \
            if (g_ == 1) BODY(1, 16); else if (g_ == 2) BODY(2, 16);  \
            else if (g_ == 3) BODY(3, 16); else BODY(4, 16);          \
        } else if (lpr_ == 32) {                                      \
            if (g_ == 1) BODY(1, 32); else if (g_ == 2) BODY(2, 32);  \
            else if (g_ == 3) BODY(3, 32); else BODY(4, 32);          \
        } else {                                                      \
            if (g_ == 1) BODY(1, 64); else if (g_ == 2) BODY(2, 64);  \
            else if (g_ == 3) BODY(3, 64); else BODY(4, 64);          \
        }                                                             \
    } while (0)

// Picks of one pass (uniform across the wave): pick[t] for t < nt, the last
// valid pick repeated above (its results are dropped).
// With DIRECT (one-token batches, no sort) position p is pick p itself.
template <int NT, bool DIRECT = false>
__device__ __forceinline__ void pass_picks(const int32_t* __restrict__ pair_list, int p, int nt, int (&pick)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) pick[t] = DIRECT ? p + min(t, nt - 1) : pair_list[p + min(t, nt - 1)];
}

template <int F, int NT, int NCHG, bool DIRECT>
__device__ __forceinline__ void gu_pass(const RowPtrs<2 * Fmt<F>::RGU>& rp, const SlabView& sv, const unsigned char* slab,
                                        const ActRows& ar, const int32_t* __restrict__ pair_list, int p, int nt,
                                        int H, int I, int k, int r_base, const float* __restrict__ xscale,
                                        void* __restrict__ hbuf) {
    using Acc = typename Fmt<F>::Acc;
    constexpr int ROWS = 2 * Fmt<F>::RGU;  // gate rows, then the same up rows
    constexpr int V = ROWS * NT;
    const int lane = threadIdx.x & 63;
    int pick[NT], tok[NT];
    pass_picks<NT, DIRECT>(pair_list, p, nt, pick);
#pragma unroll
    for (int t = 0; t < NT; ++t) tok[t] = pick[t] / k;
    Acc acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0;
    gemv_rows<F, ROWS, NT, NCHG, 64, DIRECT>(rp, ar, tok, H / Fmt<F>::EPG, lane, acc);
    int idx;
    Acc v = moe::wave_multi_sum<V>(acc, lane, idx);
    const Acc up = __shfl_xor(v, 32, 64);
    if (moe::multi_sum_holder<V>(lane) && !(lane & 32)) {
        const int r = idx / NT, t = idx % NT;
        const int row = r_base + r;
        if (row < I && t < nt) {
            const int pk = pick[t];
            if constexpr (F == MOE_W_W8A8) {
                const float sx = xscale[tok[t]];
                const float sg = reinterpret_cast<const float*>(slab + sv.s0)[row];
                const float su = reinterpret_cast<const float*>(slab + sv.s1)[row];
                const float g = ((float)v * sx) * sg;
                const float u = ((float)up * sx) * su;
                const double hd = ((double)g / (1.0 + exp(-(double)g))) * (double)u;
                reinterpret_cast<float*>(hbuf)[(int64_t)pk * I + row] = (float)hd;
            } else {
                const float g = (float)v, u = (float)up;
                const float h = g / (1.0f + expf(-g)) * u;
                if constexpr (F == MOE_W_F32) reinterpret_cast<float*>(hbuf)[(int64_t)pk * I + row] = h;
                else reinterpret_cast<uint16_t*>(hbuf)[(int64_t)pk * I + row] = moe::f32_to_bf16(h);
            }
        }
    }
}

// Token passes of up to NTMAX tokens; the body is instantiated for the
// smallest power of two that holds the pass's tokens.
constexpr int NT_TOP = NTMAX > 4 ? NTMAX : 4;
#define MOE_NT_DISPATCH(nt, BODY)              \
    do {                                       \
        if ((nt) <= 1) { BODY(1); }            \
        else if ((nt) <= 2) { BODY(2); }       \
        else if ((nt) <= 4 || NTMAX <= 4) { BODY(4); } \
        else { BODY(NT_TOP); }                 \
    } while (0)

// One workgroup per (slot with work, tile of 4 * RGU gate rows and the
// same up rows); each wave owns RGU gate and RGU up rows.  Waves are
// independent: no LDS, no barrier.
// DIRECT (one-token batches): no pick sort; workgroup group a takes pick a
// (slot slot_ids[a]), which needs no list: a token's picks are distinct
// experts, and a pick taken alone is right in any case.
template <int F, int NCHG, bool DIRECT>
__global__ void __launch_bounds__(FFN_THREADS) k_gu(SlabView sv, const void* __restrict__ act,
                                                    const float* __restrict__ xscale, const float* __restrict__ xbsum,
                                                    int H, int I, int k, const int32_t* __restrict__ slot_off,
                                                    const int32_t* __restrict__ pair_list,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, void* __restrict__ hbuf,
                                                    int tiles, const int32_t* __restrict__ slot_ids, int S) {
    constexpr int RPW_GU = Fmt<F>::RGU;
    constexpr int ROWS = 2 * RPW_GU;
    const int tiles_l = (tiles + Fmt<F>::REP - 1) / Fmt<F>::REP;  // workgroups per slot
    const int a = blockIdx.x / tiles_l;
    int s;
    if constexpr (DIRECT) {
        s = slot_ids[a];
        if (s < 0 || s >= S) return;
    } else {
        if (a >= *n_active) return;
        s = active[a];
    }
    const unsigned char* slab = sv.slots + (size_t)s * sv.slab_bytes;
#pragma unroll
    for (int rep = 0; rep < Fmt<F>::REP; ++rep) {
    const int tile = blockIdx.x % tiles_l + rep * tiles_l;
    if (tile >= tiles) break;
    const int r_base = tile * (4 * RPW_GU) + (threadIdx.x >> 6) * RPW_GU;
    const int KG = H / Fmt<F>::EPG;
    const size_t row_bytes = (size_t)KG * 16;
    RowPtrs<ROWS> rp;
#pragma unroll
    for (int r = 0; r < RPW_GU; ++r) {
        const int row = min(r_base + r, I - 1);
        rp.w[r] = slab + sv.w0 + row * row_bytes;
        rp.w[RPW_GU + r] = slab + sv.w1 + row * row_bytes;
        rp.s[r] = slab + sv.s0 + (size_t)row * KG * 2;
        rp.s[RPW_GU + r] = slab + sv.s1 + (size_t)row * KG * 2;
    }
    const ActRows ar{reinterpret_cast<const unsigned char*>(act), (size_t)H * Fmt<F>::ABYTES, xbsum};
    const int p0 = DIRECT ? a : slot_off[s], ns = DIRECT ? 1 : slot_off[s + 1] - p0;
    (void)ns;
    // passes of up to NTMAX tokens (a slot with more tokens re-reads its rows)
#define MOE_GU(N) gu_pass<F, N, NCHG, DIRECT>(rp, sv, slab, ar, pair_list, p0 + c0, nt, H, I, k, r_base, xscale, hbuf)
    if constexpr (DIRECT) {  // one pick
        const int c0 = 0, nt = 1;
        MOE_GU(1);
    } else {
        for (int c0 = 0; c0 < ns; c0 += NTMAX) {
            const int nt = min(NTMAX, ns - c0);
            MOE_NT_DISPATCH(nt, MOE_GU);
        }
    }
#undef MOE_GU
    }
}

template <int F, int NT, int NCHG, int LPR>
__device__ __forceinline__ void down_pass(const RowPtrs<Fmt<F>::RDN>& rp, const SlabView& sv, const unsigned char* slab,
                                          const ActRows& ar, const int32_t* __restrict__ pair_list, int p, int nt,
                                          int H, int I, int r_base, const float* __restrict__ hscale,
                                          const float* __restrict__ wts, float* __restrict__ part) {
    using Acc = typename Fmt<F>::Acc;
    constexpr int RPI = 64 / LPR;
    constexpr int RPW_DN = Fmt<F>::RDN;
    constexpr int V = (RPW_DN / RPI) * NT;  // values per lane
    static_assert(V <= LPR, "a lane group reduces at most LPR values at once");
    const int lane = threadIdx.x & 63;
    int pick[NT];
    pass_picks<NT>(pair_list, p, nt, pick);
    Acc acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0;
    gemv_rows<F, RPW_DN, NT, NCHG, LPR>(rp, ar, pick, I / Fmt<F>::EPG, lane, acc);
    // reduce inside each group of LPR lanes (strides LPR/2 .. 1)
    int idx = 0;
    moe::multi_sum_level<V, LPR / 2>(acc, lane, idx);
    const Acc v = acc[0];
    if ((lane & (LPR / V - 1)) == 0) {
        const int i = idx / NT, t = idx % NT;
        const int row = r_base + lane / LPR + RPI * i;
        if (row < H && t < nt) {
            const int pk = pick[t];
            float o;
            if constexpr (F == MOE_W_W8A8)
                o = ((float)v * hscale[pk]) * reinterpret_cast<const float*>(slab + sv.s0)[row];
            else
                o = (float)v;
            part[(int64_t)pk * H + row] = wts[pk] * o;
        }
    }
}

template <int F, int NCHG, int LPR>
__global__ void __launch_bounds__(FFN_THREADS) k_down(SlabView sv, const void* __restrict__ hact,
                                                      const float* __restrict__ hscale,
                                                      const float* __restrict__ hbsum, const float* __restrict__ wts,
                                                      int H, int I, const int32_t* __restrict__ slot_off,
                                                      const int32_t* __restrict__ pair_list,
                                                      const int32_t* __restrict__ active,
                                                      const int32_t* __restrict__ n_active, float* __restrict__ part,
                                                      int tiles) {
    constexpr int RPW_DN = Fmt<F>::RDN;
    const int tiles_l = (tiles + Fmt<F>::REP - 1) / Fmt<F>::REP;  // workgroups per slot
    const int a = blockIdx.x / tiles_l;
    if (a >= *n_active) return;
    const int s = active[a];
    const unsigned char* slab = sv.slots + (size_t)s * sv.slab_bytes;
#pragma unroll
    for (int rep = 0; rep < Fmt<F>::REP; ++rep) {
    const int tile = blockIdx.x % tiles_l + rep * tiles_l;
    if (tile >= tiles) break;
    const int r_base = tile * (4 * RPW_DN) + (threadIdx.x >> 6) * RPW_DN;
    const int KG = I / Fmt<F>::EPG;
    const size_t row_bytes = (size_t)KG * 16;
    RowPtrs<RPW_DN> rp;
#pragma unroll
    for (int r = 0; r < RPW_DN; ++r) {
        const int row = min(r_base + r, H - 1);
        rp.w[r] = slab + sv.w0 + row * row_bytes;
        rp.s[r] = slab + sv.s0 + (size_t)row * KG * 2;
    }
    const ActRows ar{reinterpret_cast<const unsigned char*>(hact), (size_t)I * Fmt<F>::ABYTES, hbsum};
    const int p0 = slot_off[s], ns = slot_off[s + 1] - p0;
    for (int c0 = 0; c0 < ns; c0 += NTMAX) {
        const int nt = min(NTMAX, ns - c0);
#define MOE_DN(N) \
    down_pass<F, N, NCHG, LPR>(rp, sv, slab, ar, pair_list, p0 + c0, nt, H, I, r_base, hscale, wts, part)
        MOE_NT_DISPATCH(nt, MOE_DN);
#undef MOE_DN
    }
    }
}

// One token's down projection and reduction in one launch (fp32, bf16,
// 4-bit): workgroup b takes output rows [RDN b, RDN b + RDN) for every pick of
// the token, the four waves splitting the picks (pick j to wave j % 4); each
// wave's dot products are those of k_down for one pick (same lanes, same
// order, block sums made here), w_j * o_j is staged in LDS and the rows are
// summed over the resident picks in pick order from +0.0, as k_reduce does,
// so y has the bits of k_down followed by k_reduce.
template <int F, int NCHG, int LPR>
__global__ void __launch_bounds__(FFN_THREADS) k_down_tok(SlabView sv, const void* __restrict__ hact,
                                                          const float* __restrict__ wts, int H, int I, int k, int S,
                                                          const int32_t* __restrict__ slot_ids,
                                                          float* __restrict__ y) {
    constexpr int RPW_DN = Fmt<F>::RDN;
    constexpr int RPI = 64 / LPR;
    constexpr int V = RPW_DN / RPI;  // values per lane: one token
    static_assert(F != MOE_W_W8A8, "int8 h needs its codes");
    __shared__ float cpart[MOE_MAX_K][RPW_DN];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int r_base = blockIdx.x * RPW_DN;
    const int KG = I / Fmt<F>::EPG;
    const size_t row_bytes = (size_t)KG * 16;
    const ActRows ar{reinterpret_cast<const unsigned char*>(hact), (size_t)I * Fmt<F>::ABYTES, nullptr};
    for (int j = wid; j < k; j += 4) {
        const int s = slot_ids[j];
        if (s < 0 || s >= S) continue;  // the whole wave
        const unsigned char* slab = sv.slots + (size_t)s * sv.slab_bytes;
        RowPtrs<RPW_DN> rp;
#pragma unroll
        for (int r = 0; r < RPW_DN; ++r) {
            const int row = min(r_base + r, H - 1);
            rp.w[r] = slab + sv.w0 + row * row_bytes;
            rp.s[r] = slab + sv.s0 + (size_t)row * KG * 2;
        }
        typename Fmt<F>::Acc acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0;
        const int pick[1] = {j};
        gemv_rows<F, RPW_DN, 1, NCHG, LPR, true>(rp, ar, pick, KG, lane, acc);
        int idx = 0;
        moe::multi_sum_level<V, LPR / 2>(acc, lane, idx);
        if ((lane & (LPR / V - 1)) == 0) cpart[j][lane / LPR + RPI * idx] = wts[j] * (float)acc[0];
    }
    __syncthreads();
    if (threadIdx.x < RPW_DN && r_base + (int)threadIdx.x < H) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int s = slot_ids[j];
            if (s >= 0 && s < S) acc += cpart[j][threadIdx.x];
        }
        y[r_base + threadIdx.x] = acc;
    }
}

// Per-block sums of rows of bf16 activations, for 4-bit weights: out[r][b] =
// sum of row r's inputs 32b .. 32b+31 (block_sum_bf16).  The block is read as
// four 16-byte loads that do not wait for the row's `valid` entry (in bounds
// either way; a skipped row's sum is not stored).
__global__ void __launch_bounds__(256) k_block_sums(const uint16_t* __restrict__ src, int rows, int len,
                                                    const int32_t* __restrict__ valid, float* __restrict__ out) {
    const int nb = len / 32;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)rows * nb) return;
    const int r = (int)(i / nb), b = (int)(i % nb);
    const bool ok = !valid || valid[r] >= 0;
    const v4u* p = reinterpret_cast<const v4u*>(src + (int64_t)r * len + 32 * b);
    const float sum = block_sum_bf16(p[0], p[1], p[2], p[3]);
    if (ok) out[i] = sum;
}

// y[t][m] = sum_j part[t*k+j][m] over resident picks, j ascending; +0.0 if none.
// The picks' rows are loaded eight at a time before any is added, and their
// addresses do not wait for the slot ids (the row of a non-resident pick is
// read, in bounds, and not added), so a thread waits on one round of loads
// per eight picks, not on the ids and then the rows.
__global__ void __launch_bounds__(256) k_reduce(const float* __restrict__ part, const int32_t* __restrict__ slot_ids,
                                                int T, int k, int S, int H, float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
    const int h4 = H / 4;
    if (i >= (int64_t)T * h4) return;
    const int t = (int)(i / h4), m4 = (int)(i % h4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 v[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int sl = j < k ? slot_ids[t * k + j] : -1;
            ok[u] = sl >= 0 && sl < S;
            const int64_t row = (int64_t)t * k + (j < k ? j : 0);
            v[u] = reinterpret_cast<const float4*>(part + row * H)[m4];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (ok[u]) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
        }
    }
    reinterpret_cast<float4*>(y + (int64_t)t * H)[m4] = acc;
}

// k_reduce for the bf16 partials of the prefill-shaped kernels: each thread
// sums eight columns (16 bytes of each pick's row) in fp32, picks in top-k
// order as k_reduce, and stores them as two float4.
__global__ void __launch_bounds__(256) k_reduce16(const uint16_t* __restrict__ part,
                                                  const int32_t* __restrict__ slot_ids, int T, int k, int S, int H,
                                                  float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of an 8-column group
    const int h8 = H / 8;
    if (i >= (int64_t)T * h8) return;
    const int t = (int)(i / h8), m8 = (int)(i % h8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
        v4u v[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int sl = j < k ? slot_ids[t * k + j] : -1;
            ok[u] = sl >= 0 && sl < S;
            const int64_t row = (int64_t)t * k + (j < k ? j : 0);
            v[u] = reinterpret_cast<const v4u*>(part + row * H)[m8];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (ok[u]) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc[2 * c] += __uint_as_float(v[u][c] << 16);
                    acc[2 * c + 1] += __uint_as_float(v[u][c] & 0xffff0000u);
                }
            }
        }
    }
    float4* yr = reinterpret_cast<float4*>(y + (int64_t)t * H) + 2 * m8;
    yr[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    yr[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

__global__ void __launch_bounds__(256) k_combine(float* __restrict__ y, const float* __restrict__ y_add, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = y[i] + y_add[i];
}

template <int F>
int run_ffn(const void* x, const int32_t* slot_ids, const float* w, int T, int k, const void* slot_store,
            size_t slab_bytes, int S, int H, int I, float* y, unsigned char* ws, const WsLayout& L,
            const moe_slab_layout_t& lay, hipStream_t st) {
    const int P = T * k;
    int32_t* slot_off = reinterpret_cast<int32_t*>(ws + L.slot_off);
    int32_t* pair_list = reinterpret_cast<int32_t*>(ws + L.pair_list);
    int32_t* active = reinterpret_cast<int32_t*>(ws + L.active);
    int32_t* n_active = reinterpret_cast<int32_t*>(ws + L.n_active);
    void* hbuf = ws + L.h;
    float* part = reinterpret_cast<float*>(ws + L.part);
    int rc;
    // bf16 batches of PF_MIN_P picks or more, and int8 batches of PF_MIN_P_I8 or more, run on the MFMA grouped GEMMs;
    // the sort writes their tile list
    const bool use_pf = ((F == MOE_W_BF16 && P >= PF_MIN_P) || (F == MOE_W_W8A8 && P >= PF_MIN_P_I8)) &&
                        moe_pf_supported(F, H, I);
    const int pf_mt = moe_pf_tile_rows_for(F, T, k, S, H, I);
    moe_pf_tile* pf_tiles = use_pf ? reinterpret_cast<moe_pf_tile*>(ws + L.pf_tiles) : nullptr;
    int32_t* pf_n_tiles = use_pf ? reinterpret_cast<int32_t*>(ws + L.pf_tiles + (size_t)moe_pf_max_tiles(T, k, S) *
                                                                                     sizeof(moe_pf_tile))
                                 : nullptr;

    // decode-sized bf16 batches: the gate/up GEMM sorts the picks itself
    const bool fused_sort = F == MOE_W_BF16 && use_pf && moe_pf_fused_sort(T, k);
    // int8 matrix-core path: per gate/up column tile and pick, the max |h|
    float* hmax = (F == MOE_W_W8A8 && use_pf) ? reinterpret_cast<float*>(ws + L.hmax) : nullptr;
    // one token on the row-streaming kernels (int8 aside, whose x codes the
    // sort launch makes): no sort, each gate/up and down workgroup takes one
    // pick (slot_work), and 4-bit block sums are made by those kernels
    const bool direct = T == 1 && !use_pf && F != MOE_W_W8A8;
    // quantised batches sorted by one workgroup: x prepared in the same launch
    int xprep = XPREP_NONE;
    if (P <= GROUP_MULTI_P && !direct) {
        if constexpr (F == MOE_W_W8A8) xprep = XPREP_I8;
        if constexpr (F == MOE_W_Q4B32) xprep = XPREP_BSUM;
    }
    if (direct || fused_sort) {
        // no sort launch: the gate/up workgroups write the pick and tile lists
        // (fused sort) or take one pick each (direct)
    } else if (P > GROUP_MULTI_P) {
        const int nch = (P + GROUP_THREADS - 1) / GROUP_THREADS;
        int32_t* gcnt = reinterpret_cast<int32_t*>(ws + L.gcnt);
        hipLaunchKernelGGL(k_group_hist, dim3(nch), dim3(GROUP_THREADS), 0, st, slot_ids, P, S, gcnt);
        if ((rc = moe_check_launch("moe_ffn_slots/group_hist"))) return rc;
        hipLaunchKernelGGL(k_group_place, dim3(nch), dim3(GROUP_THREADS), 0, st, slot_ids, P, S, gcnt, nch, slot_off,
                           pair_list, active, n_active, pf_tiles, pf_n_tiles, pf_mt);
        if ((rc = moe_check_launch("moe_ffn_slots/group_place"))) return rc;
    } else if (P <= GROUP_SMALL_P && xprep == XPREP_NONE && !use_pf) {
        hipLaunchKernelGGL(k_group_small, dim3(1), dim3(64), 0, st, slot_ids, P, S, slot_off, pair_list, active,
                           n_active);
        if ((rc = moe_check_launch("moe_ffn_slots/group_small"))) return rc;
    } else {
        hipLaunchKernelGGL(k_group, dim3(1 + x_prep_wgs(xprep, T, H)), dim3(GROUP_THREADS), 0, st, slot_ids, P, S,
                           slot_off, pair_list, active, n_active, pf_tiles, pf_n_tiles, pf_mt, xprep,
                           reinterpret_cast<const uint16_t*>(x), T, H,
                           reinterpret_cast<int8_t*>(ws + L.xq), reinterpret_cast<float*>(ws + L.xs),
                           reinterpret_cast<float*>(ws + L.xbs));
        if ((rc = moe_check_launch("moe_ffn_slots/group"))) return rc;
    }

    if (use_pf) {
        const void* act = x;
        const float* xs = nullptr;
        if constexpr (F == MOE_W_W8A8) {
            act = ws + L.xq;
            xs = reinterpret_cast<const float*>(ws + L.xs);
            if (!xprep) {  // the sort ran as hist + place: x's codes in a launch of their own
                hipLaunchKernelGGL((k_quant_rows<true>), dim3(T), dim3(256), 0, st, x, H, (const int32_t*)nullptr,
                                   reinterpret_cast<int8_t*>(ws + L.xq), reinterpret_cast<float*>(ws + L.xs));
                if ((rc = moe_check_launch("moe_ffn_slots/quant_x"))) return rc;
            }
        }
        rc = moe_pf_run(act, w, T, k, slot_store, slab_bytes, S, H, I, lay, pair_list, ws + L.pf_tiles, hbuf, part,
                        st, fused_sort ? slot_ids : nullptr, F, xs, hmax);
        if (rc) return rc;
        if (moe_pf_part_bf16(F, T, k)) {  // prefill-shaped kernels: bf16 partials
            const int64_t n8 = (int64_t)T * (H / 8);
            hipLaunchKernelGGL(k_reduce16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                               reinterpret_cast<const uint16_t*>(part), slot_ids, T, k, S, H, y);
            return moe_check_launch("moe_ffn_slots/reduce16");
        }
        const int64_t n4 = (int64_t)T * (H / 4);
        hipLaunchKernelGGL(k_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, slot_ids, T, k, S,
                           H, y);
        return moe_check_launch("moe_ffn_slots/reduce");
    }

    const void* gu_act = x;
    const float* xscale = nullptr;
    const float* xbsum = nullptr;
    if constexpr (F == MOE_W_W8A8) {
        int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
        float* xs = reinterpret_cast<float*>(ws + L.xs);
        if (!xprep) {
            hipLaunchKernelGGL((k_quant_rows<true>), dim3(T), dim3(256), 0, st, x, H, (const int32_t*)nullptr, xq,
                               xs);
            if ((rc = moe_check_launch("moe_ffn_slots/quant_x"))) return rc;
        }
        gu_act = xq;
        xscale = xs;
    }
    if constexpr (F == MOE_W_Q4B32) {
        float* xbs = reinterpret_cast<float*>(ws + L.xbs);
        if (!xprep && !direct) {
            const int64_t n = (int64_t)T * (H / 32);
            hipLaunchKernelGGL(k_block_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               reinterpret_cast<const uint16_t*>(x), T, H, (const int32_t*)nullptr, xbs);
            if ((rc = moe_check_launch("moe_ffn_slots/block_sums_x"))) return rc;
        }
        xbsum = direct ? nullptr : xbs;
    }

    SlabView gv{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1], lay.s[0], lay.s[1]};
    const int tiles_gu = (I + 4 * Fmt<F>::RGU - 1) / (4 * Fmt<F>::RGU);
    // at most min(S, P) slots have work: workgroups beyond them would only read n_active and leave
    const int max_active = S < P ? S : P;
#define MOE_LAUNCH_GU_(G, D)                                                                                  \
    hipLaunchKernelGGL((k_gu<F, G, D>), dim3(max_active * ((tiles_gu + Fmt<F>::REP - 1) / Fmt<F>::REP)),          \
                       dim3(FFN_THREADS), 0, st, gv, gu_act, xscale, xbsum, H, I, k, slot_off, pair_list, active,  \
                       n_active, hbuf, tiles_gu, slot_ids, S)
#define MOE_LAUNCH_GU(G)                                                    \
    if (direct) {                                                           \
        if constexpr (F != MOE_W_W8A8) MOE_LAUNCH_GU_(G, true);             \
    } else                                                                  \
        MOE_LAUNCH_GU_(G, false)
    MOE_NCHG_DISPATCH(H / Fmt<F>::EPG, MOE_LAUNCH_GU);
#undef MOE_LAUNCH_GU
#undef MOE_LAUNCH_GU_
    if ((rc = moe_check_launch("moe_ffn_slots/gate_up"))) return rc;

    const void* dn_act = hbuf;
    const float* hscale = nullptr;
    const float* hbsum = nullptr;
    if constexpr (F == MOE_W_W8A8) {
        int8_t* hq = reinterpret_cast<int8_t*>(ws + L.hq);
        float* hsc = reinterpret_cast<float*>(ws + L.hs);
        hipLaunchKernelGGL((k_quant_rows<false>), dim3(P), dim3(256), 0, st, hbuf, I, slot_ids, hq, hsc);
        if ((rc = moe_check_launch("moe_ffn_slots/quant_h"))) return rc;
        dn_act = hq;
        hscale = hsc;
    }
    if constexpr (F == MOE_W_Q4B32) {
        if (!direct) {  // one token: the down kernel sums its blocks itself
            float* hbs = reinterpret_cast<float*>(ws + L.hbs);
            const int64_t n = (int64_t)P * (I / 32);
            hipLaunchKernelGGL(k_block_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               reinterpret_cast<const uint16_t*>(hbuf), P, I, slot_ids, hbs);
            if ((rc = moe_check_launch("moe_ffn_slots/block_sums_h"))) return rc;
            hbsum = hbs;
        }
    }
    SlabView dv{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0, lay.s[2], 0};
    if constexpr (F != MOE_W_W8A8) {
        if (direct) {  // one token: down projection and reduction in one launch
#define MOE_LAUNCH_DT(G, LP)                                                                                       \
    hipLaunchKernelGGL((k_down_tok<F, G, LP>), dim3((H + Fmt<F>::RDN - 1) / Fmt<F>::RDN), dim3(FFN_THREADS), 0, st, \
                       dv, dn_act, w, H, I, k, S, slot_ids, y)
            MOE_DOWN_DISPATCH(I / Fmt<F>::EPG, MOE_LAUNCH_DT);
#undef MOE_LAUNCH_DT
            return moe_check_launch("moe_ffn_slots/down_token");
        }
    }
    const int tiles_dn = (H + 4 * Fmt<F>::RDN - 1) / (4 * Fmt<F>::RDN);
#define MOE_LAUNCH_DN(G, LP)                                                                                 \
    hipLaunchKernelGGL((k_down<F, G, LP>), dim3(max_active * ((tiles_dn + Fmt<F>::REP - 1) / Fmt<F>::REP)),     \
                       dim3(FFN_THREADS), 0, st, dv, dn_act, hscale, hbsum, w, H, I, slot_off, pair_list, active, \
                       n_active, part, tiles_dn)
    MOE_DOWN_DISPATCH(I / Fmt<F>::EPG, MOE_LAUNCH_DN);
#undef MOE_LAUNCH_DN
    if ((rc = moe_check_launch("moe_ffn_slots/down"))) return rc;

    const int64_t n4 = (int64_t)T * (H / 4);
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, slot_ids, T, k, S, H, y);
    return moe_check_launch("moe_ffn_slots/reduce");
}

// ------------------------------------------------ allocation-free entry

// `scratch` (the workspace of moe_ffn_slots_noalloc) is declared at the top
// of this file.

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex scratch_mu;
unsigned char* scratch_dev[NOALLOC_MAX_DEVICES];  // device address of `scratch` per device, once looked up

// The current device's copy of the scratch array (looked up on the first
// call on that device, with the device current).
int scratch_for_current_device(unsigned char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        (void)hipGetLastError();
        return moe_fail(MOE_E_HIP, "moe_ffn_slots_noalloc: no current device (%s) or device %d beyond %d",
                        hipGetErrorString(e), dev, NOALLOC_MAX_DEVICES - 1);
    }
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_HIP, "moe_ffn_slots_noalloc: cannot find the scratch array on device %d (%s)", dev,
                            hipGetErrorString(e));
        }
        scratch_dev[dev] = reinterpret_cast<unsigned char*>(p);
    }
    *out = scratch_dev[dev];
    return MOE_OK;
}

// Argument checks shared by both entry points; the workspace layout on success.
int ffn_check(const void* x, int x_dtype, const int32_t* slot_ids, const float* w, int T, int k,
              const void* slot_store, size_t slab_bytes, int S, int w_type, int H, int I, float* y,
              moe_slab_layout_t* lay, const char* who) {
    MOE_REQUIRE(T >= 0 && k >= 1 && k <= MOE_MAX_K && S >= 1 && H >= 1 && I >= 1, MOE_E_ARG,
                "%s: T=%d k=%d S=%d H=%d I=%d out of range", who, T, k, S, H, I);
    MOE_REQUIRE(S <= MOE_MAX_S, MOE_E_SHAPE, "%s: S=%d exceeds %d", who, S, MOE_MAX_S);
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(x && slot_ids && w && slot_store && y, MOE_E_ARG,
                "%s: x, slot_ids, w, slot_store and y must be non-NULL", who);
    int rc = moe_layout(w_type, H, I, lay);
    if (rc) return rc;
    MOE_REQUIRE(slab_bytes >= (size_t)lay->total && slab_bytes % 16 == 0, MOE_E_ALIGN,
                "%s: slab_bytes=%zu must be a 16-byte multiple >= %lld", who, slab_bytes, (long long)lay->total);
    MOE_REQUIRE(moe_aligned16(slot_store) && moe_aligned16(x) && moe_aligned16(y), MOE_E_ALIGN,
                "%s: x, slot_store and y must be 16-byte aligned", who);
    const int want_x = w_type == MOE_W_F32 ? MOE_X_F32 : MOE_X_BF16;
    MOE_REQUIRE(x_dtype == want_x, MOE_E_DTYPE, "%s: weight format %d needs activation format %d, got %d", who,
                w_type, want_x, x_dtype);
    return MOE_OK;
}

int ffn_dispatch(const void* x, const int32_t* slot_ids, const float* w, int T, int k, const void* slot_store,
                 size_t slab_bytes, int S, int w_type, int H, int I, float* y, unsigned char* wsb,
                 const WsLayout& L, const moe_slab_layout_t& lay, hipStream_t stream) {
    switch (w_type) {
        case MOE_W_F32:
            return run_ffn<MOE_W_F32>(x, slot_ids, w, T, k, slot_store, slab_bytes, S, H, I, y, wsb, L, lay, stream);
        case MOE_W_BF16:
            return run_ffn<MOE_W_BF16>(x, slot_ids, w, T, k, slot_store, slab_bytes, S, H, I, y, wsb, L, lay, stream);
        case MOE_W_W8A8:
            return run_ffn<MOE_W_W8A8>(x, slot_ids, w, T, k, slot_store, slab_bytes, S, H, I, y, wsb, L, lay, stream);
        case MOE_W_Q4B32:
            return run_ffn<MOE_W_Q4B32>(x, slot_ids, w, T, k, slot_store, slab_bytes, S, H, I, y, wsb, L, lay, stream);
        default:
            return moe_fail(MOE_E_DTYPE, "moe_ffn_slots: unknown weight format %d", w_type);
    }
}

}  // namespace

extern "C" {

size_t moe_ffn_workspace_bytes(int T, int k, int S, int w_type, int H, int I) {
    if (T < 0 || k < 1 || S < 1 || H < 1 || I < 1) return 0;
    return ws_layout(T, k, S, w_type, H, I).total;
}

int moe_ffn_slots(const void* x, int x_dtype, const int32_t* slot_ids, const float* w, int T, int k,
                  const void* slot_store, size_t slab_bytes, int S, int w_type, int H, int I, float* y, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
    moe_slab_layout_t lay;
    int rc = ffn_check(x, x_dtype, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y, &lay,
                       "moe_ffn_slots");
    if (rc || T == 0) return rc ? rc : moe_ok();
    MOE_REQUIRE(ws && moe_aligned16(ws), MOE_E_ARG, "moe_ffn_slots: ws must be non-NULL and 16-byte aligned");
    const WsLayout L = ws_layout(T, k, S, w_type, H, I);
    MOE_REQUIRE(ws_bytes >= L.total, MOE_E_ARG, "moe_ffn_slots: workspace of %zu bytes, need %zu", ws_bytes, L.total);
    return ffn_dispatch(x, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y,
                        reinterpret_cast<unsigned char*>(ws), L, lay, stream);
}

int moe_ffn_slots_noalloc(const void* x, int x_dtype, const int32_t* slot_ids, const float* w, int T, int k,
                          const void* slot_store, size_t slab_bytes, int S, int w_type, int H, int I, float* y,
                          hipStream_t stream) {
    moe_slab_layout_t lay;
    int rc = ffn_check(x, x_dtype, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y, &lay,
                       "moe_ffn_slots_noalloc");
    if (rc || T == 0) return rc ? rc : moe_ok();
    const WsLayout L = ws_layout(T, k, S, w_type, H, I);
    MOE_REQUIRE(L.total <= NOALLOC_SCRATCH_BYTES, MOE_E_SHAPE,
                "moe_ffn_slots_noalloc: T=%d k=%d S=%d H=%d I=%d needs %zu bytes of workspace; the static scratch "
                "holds %zu (use moe_ffn_slots with a workspace of your own)",
                T, k, S, H, I, L.total, NOALLOC_SCRATCH_BYTES);
    unsigned char* ws = nullptr;
    if ((rc = scratch_for_current_device(&ws))) return rc;
    return ffn_dispatch(x, slot_ids, w, T, k, slot_store, slab_bytes, S, w_type, H, I, y, ws, L, lay, stream);
}

size_t moe_ffn_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int moe_combine(float* y, const float* y_add, int T, int H, hipStream_t stream) {
    MOE_REQUIRE(y && y_add && T >= 0 && H >= 1, MOE_E_ARG, "moe_combine: bad arguments");
    const int64_t n = (int64_t)T * H;
    if (n == 0) return moe_ok();
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y, y_add, n);
    return moe_check_launch("moe_combine");
}

}  // extern "C"

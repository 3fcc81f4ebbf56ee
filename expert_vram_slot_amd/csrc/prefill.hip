// Grouped SwiGLU expert FFN for prefill-sized token groups, bf16 weights, on
// the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Same computation as the decode path (sozai.app transcript
// "rtx-3060-run-35b-llamacpp", "Full Transcript": resident experts on the
// GPU, zero for the rest; "Porting vllm-expert-cache to NVIDIA GPUs", "What
// this package does": the expert FFN runs in slot space), arranged as grouped
// GEMMs once a slot holds tens of tokens:
//
//   k_group      picks sorted by slot (shared with the decode path), and the
//                list of (slot, up to PF_MT consecutive picks) tiles; batches
//                of at most 1024 picks on decode-shaped tiles skip it (the
//                gate/up kernel groups the picks itself, dec_sort_tile)
//   k_pf_gemm<GU>   [g | u] = X_s [W_g; W_u]^T per tile of 64 h columns,
//                   SwiGLU epilogue, h (bf16, RNE) stored in sorted-pick order
//   k_pf_gemm<DOWN> O = H_s W_d^T per tile of 128 output columns,
//                   part[pick] = w * O (bf16, RNE; the decode-shaped
//                   kernels keep fp32 partials)
//   k_dec_gemm<GU|DOWN>  the same two GEMMs on decode-shaped tiles
//   k_pf_wide<GU|DOWN>   the same two GEMMs on 256 x 256 tiles when slots
//                        hold hundreds of picks
//   k_reduce16   y[t] = fp32 sum of the bf16 partials of its resident picks
//                in top-k order (k_reduce, the decode path's, sums fp32 ones)
//
// Prefill-sized batches (4096 picks and more): a workgroup owns PF_MT = 128
// token rows x NB * 32 weight rows (NB = 8 when H is a multiple of 256, else 4)
// and walks K in steps of 64.
// Decode-sized batches (a few picks per slot) use k_dec_gemm below: 32 token
// rows, each wave a 32-row weight block.  Each k-step is fetched into
// registers two steps ahead and stored to one of two LDS buffers; 16-byte
// chunks are XOR-swizzled per row
// so that both the stores and the MFMA operand reads are free of bank
// conflicts.  Each wave owns 32 of the token rows; a wave whose rows are all
// past the tile's picks skips its MFMAs.  Workgroups that share a tile's
// token rows are placed on one XCD (workgroups go to XCDs round-robin by
// index), so those rows are fetched from HBM once and then served by that
// XCD's L2.  Every weight row is read by exactly one workgroup per tile.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "prefill.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
using v4u = uint32_t __attribute__((ext_vector_type(4)));

constexpr int PF_THREADS = 256;
constexpr int PF_MT = 128;         // token rows per prefill-shaped tile
constexpr int PF_KT = 64;          // k per step (128 bytes of bf16 per row)
constexpr int PF_ROWB = PF_KT * 2; // bytes of one row of a k-step
constexpr int PF_TILE_BYTES = PF_MT * PF_ROWB;  // 16 KiB: the A tile of one k-step
// LDS of a workgroup whose B tile has NB blocks of 32 weight rows: two buffers of A and B
constexpr int pf_lds_bytes(int NB) { return 2 * (PF_TILE_BYTES + NB * 32 * PF_ROWB); }
constexpr int PF_XCD = 8;
constexpr int PF_BIG_P = 4096;  // picks from which prefill-shaped tiles are used
constexpr int PB_BIG_ROWS = 384;  // mean picks per slot from which 256-row tiles are used
constexpr int DEC_MT = 32;      // token rows of a decode-shaped tile
constexpr int DEC_NW = 4;       // waves of a decode-shaped workgroup (32 weight rows each)
constexpr int DEC_NR_GU = 2;    // register sets of k-steps in flight per thread: gate/up
constexpr int DEC_NR_DN = 2;    // and down

enum { PF_GU = 0, PF_DOWN = 1 };

// 16-byte chunk c of row r sits at chunk c ^ swz(r) of its 128-byte LDS row:
// 8 consecutive rows, and 16 consecutive rows taken with their parity, all
// land on distinct chunks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// First k-step of this workgroup's walk over the contraction.  Weight rows
// of 4 KiB (and other sizes whose steps line up across rows) read 128 B at a
// time by workgroups in lockstep put every concurrent access at the same
// offset within its row, which crowds a few HBM channels (a read probe:
// 5.3 TB/s for 4 KiB rows, 6.5 TB/s once each workgroup starts elsewhere).
// The sum over k is then taken in a rotated order, fixed per workgroup.
// Rows whose length is not a multiple of 4 KiB spread by themselves (and the
// down GEMM of the decode layer ran slower rotated), so they start at 0.
constexpr int ROT_BYTES = 4096;
__device__ __forceinline__ int k_rot(int nk) {
    return (nk * PF_ROWB) % ROT_BYTES == 0 ? (int)(blockIdx.x % (unsigned)nk) : 0;
}

using PfTile = moe_pf_tile;

struct PfArgs {
    const unsigned char* slots;  // slot store
    size_t slab_bytes;
    int64_t w0, w1;              // weight planes used (GU: gate, up; DOWN: down)
    const unsigned char* act;    // GU: x [T][H] bf16; DOWN: h [P][I] bf16 in sorted order
    const int32_t* pair_list;    // slot-sorted picks
    const float* wts;            // routing weights [P]
    const PfTile* tiles;
    const int32_t* n_tiles;
    void* out;                   // GU: h [P][I] bf16 (sorted order); DOWN: part [P][H] (bf16 in the
                                 // prefill-shaped kernels, fp32 in the decode-shaped one)
    int K;                       // contraction length (GU: H, DOWN: I)
    int N;                       // output columns (GU: I, DOWN: H)
    int k;                       // top-k (GU: token = pick / k)
    int ntiles_n;                // column tiles per token tile
    // decode gate/up only: when sort_slots is set, each workgroup sorts the
    // picks by slot itself (no separate sort launch) and the workgroups of
    // column tile 0 write the tile list and the slot-sorted pick list for the
    // down projection (into tiles_out / n_tiles_out / pair_out)
    const int32_t* sort_slots;   // [sort_P] slot id per pick (< 0: not resident)
    int sort_P, sort_S;
    int32_t* pair_out;
    PfTile* tiles_out;
    int32_t* n_tiles_out;
    // int8 weights (W8A8) only: the per-row scale planes (GU: gate, up; DOWN:
    // down) and the per-token activation scales of x (GU)
    int64_t s0, s1;
    const float* xscale;
    float* hmax;                 // [GU column tiles][P]: each tile's max |h| per pick (sorted order)
    int hstride;                 // P, the stride of hmax between column tiles
};

__device__ __forceinline__ v4u ld16(const unsigned char* p) { return *reinterpret_cast<const v4u*>(p); }

// Barrier of the two LDS buffers of a k-loop: waits for this wave's LDS
// stores and reads (lgkmcnt 0), then a bare s_barrier.  Loads from memory
// into registers stay in flight across it (a fence here would wait for every
// one of them, the ones of later k-steps too); the compiler waits for each
// where its registers are stored to LDS.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7: no wait; lgkmcnt 0
    asm volatile("s_barrier" ::: "memory");
}
__device__ __forceinline__ v4u ld16_nt(const unsigned char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}

// One workgroup's tile: QA * 32 token rows are loaded and staged (the rest of
// the 128-row tile lies past its picks), NB * 32 weight rows.
template <int MODE, int NB, int QA>
__device__ __forceinline__ void pf_gemm_tile(const PfArgs& g, const PfTile& tl, int jn, unsigned char* pf_lds) {
    constexpr int HC = NB * 16;                          // gate/up: h columns per tile
    constexpr int B_BYTES = NB * 32 * PF_ROWB;           // B tile of one k-step
    static_assert(NB >= 1 && NB <= 8, "weight blocks per wave");
    static_assert(QA >= 1 && QA <= 4, "token row blocks");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    const size_t row_bytes = (size_t)g.K * 2;

    // this thread's QA A rows and NB B rows (row = q * 32 + tid / 8, chunk tid % 8)
    const int lrow = tid >> 3, chunk = tid & 7;
    const unsigned char* arow[QA];
    const unsigned char* brow[NB];
    int soff[QA], bsoff[NB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int r = q * 32 + lrow;
        // rows past the tile's picks repeat its last row (a line the wave already reads; results dropped)
        const int pos = tl.p0 + min(r, tl.rows - 1);
        int arow_idx;
        if constexpr (MODE == PF_GU) arow_idx = g.pair_list[pos] / g.k;   // token of the pick
        else arow_idx = pos;                                             // h row in sorted order
        arow[q] = g.act + (size_t)arow_idx * row_bytes + chunk * 16;
        soff[q] = r * PF_ROWB + ((chunk ^ swz(r)) * 16);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int r = q * 32 + lrow;
        int wr;
        int64_t plane;
        if constexpr (MODE == PF_GU) {  // rows 0..HC-1 gate, HC..2HC-1 up, of h columns jn*HC ..
            plane = r < HC ? g.w0 : g.w1;
            wr = jn * HC + (r < HC ? r : r - HC);
        } else {
            plane = g.w0;
            wr = jn * (NB * 32) + r;
        }
        brow[q] = slab + plane + (size_t)wr * row_bytes + chunk * 16;
        bsoff[q] = r * PF_ROWB + ((chunk ^ swz(r)) * 16);
    }

    // operand read offsets: A row wv*32 + lane%32, B rows nb*32 + lane%32; k half = lane/32
    const int mrow = wv * 32 + (lane & 31);
    const int khalf = lane >> 5;
    int a_off[4], b_off[4][NB];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        a_off[ks] = mrow * PF_ROWB + (((ks * 2 + khalf) ^ swz(mrow)) * 16);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int r = nb * 32 + (lane & 31);
            b_off[ks][nb] = r * PF_ROWB + (((ks * 2 + khalf) ^ swz(r)) * 16);
        }
    }
    const bool active_wave = wv * 32 < tl.rows;

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[nb][x] = 0.0f;

    const int nk = g.K / PF_KT;
    v4u ra[2][QA], rb[2][NB];
    // each workgroup walks k from its own starting step (see k_rot)
    const int rot = k_rot(nk);
    auto fetch = [&](v4u (&a)[QA], v4u (&w)[NB], int kt) {
        const int kr = kt + rot;
        const size_t ko = (size_t)(kr >= nk ? kr - nk : kr) * PF_ROWB;
#pragma unroll
        for (int q = 0; q < QA; ++q) a[q] = ld16(arow[q] + ko);
#pragma unroll
        for (int q = 0; q < NB; ++q) w[q] = ld16_nt(brow[q] + ko);
    };
    auto stash = [&](const v4u (&a)[QA], const v4u (&w)[NB], int buf) {
        unsigned char* A = pf_lds + buf * (PF_TILE_BYTES + B_BYTES);
        unsigned char* B = A + PF_TILE_BYTES;
#pragma unroll
        for (int q = 0; q < QA; ++q) *reinterpret_cast<v4u*>(A + soff[q]) = a[q];
#pragma unroll
        for (int q = 0; q < NB; ++q) *reinterpret_cast<v4u*>(B + bsoff[q]) = w[q];
    };
    auto compute = [&](int buf) {
        if (!active_wave) return;
        const unsigned char* A = pf_lds + buf * (PF_TILE_BYTES + B_BYTES);
        const unsigned char* B = A + PF_TILE_BYTES;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(A + a_off[ks]));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(B + b_off[ks][nb]));
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[nb], 0, 0, 0);
            }
        }
    };

    // Two k-steps in registers ahead of the one in LDS.  nk is even (K is a
    // multiple of 128); the loop body has no branch on memory operations, so
    // each register set is waited for only where it is stored.
    fetch(ra[0], rb[0], 0);
    fetch(ra[1], rb[1], 1);
    stash(ra[0], rb[0], 0);
    lds_barrier();
    for (int kt = 0; kt + 2 < nk; kt += 2) {
        fetch(ra[0], rb[0], kt + 2);  // buffer 0 holds step kt, registers 1 hold kt + 1
        compute(0);
        stash(ra[1], rb[1], 1);
        lds_barrier();
        fetch(ra[1], rb[1], kt + 3);  // buffer 1 holds kt + 1, registers 0 hold kt + 2
        compute(1);
        stash(ra[0], rb[0], 0);
        lds_barrier();
    }
    // last two steps: buffer 0 holds nk - 2, registers 1 hold nk - 1
    compute(0);
    stash(ra[1], rb[1], 1);
    lds_barrier();
    compute(1);

    if (!active_wave) return;
    // accumulator element x of lane l: column l % 32 of block nb, row (x/4)*8 + (l/32)*4 + x%4.
    // h and the bf16 partials are stored non-temporally: the next kernel reads them from other XCDs, so
    // they gain nothing in this XCD's L2, where they would push out the weight and token lines still in
    // use (2048-token layer: 2.14 -> 2.07-2.10 ms; the same stores in the decode-shaped and the
    // large-group kernels were 1 % slower)
    const int col = lane & 31;
    if constexpr (MODE == PF_GU) {
        uint16_t* h = reinterpret_cast<uint16_t*>(g.out);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = wv * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            const size_t hrow = (size_t)(tl.p0 + r) * g.N + jn * HC;
#pragma unroll
            for (int half = 0; half < NB / 2; ++half) {
                const float gv = acc[half][x], uv = acc[NB / 2 + half][x];
                const float hv = gv / (1.0f + expf(-gv)) * uv;
                __builtin_nontemporal_store(moe::f32_to_bf16(hv), &h[hrow + half * 32 + col]);
            }
        }
    } else {
        // bf16 partials: half the bytes of the write here and of the
        // reduction's read (0.27 GB a call at 2048 tokens of the 288-expert
        // layer), one rounding of each pick's weighted row before the fp32 sum
        uint16_t* part = reinterpret_cast<uint16_t*>(g.out);
        // the pick and routing weight of each of this lane's 16 rows: all
        // loads of a kind issued together (looked up row by row behind the
        // row test, the dependent pairs serialise)
        int epk[16];
        float ewt[16];
#pragma unroll
        for (int x = 0; x < 16; ++x)
            epk[x] = g.pair_list[tl.p0 + min(wv * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3), tl.rows - 1)];
#pragma unroll
        for (int x = 0; x < 16; ++x) ewt[x] = g.wts[epk[x]];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = wv * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            uint16_t* prow = part + (size_t)epk[x] * g.N + jn * (NB * 32);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                __builtin_nontemporal_store(moe::f32_to_bf16(ewt[x] * acc[nb][x]), &prow[nb * 32 + col]);
        }
    }
}

template <int MODE, int NB>
__global__ void __launch_bounds__(PF_THREADS) k_pf_gemm(PfArgs g) {
    extern __shared__ __attribute__((aligned(16))) unsigned char pf_lds[];
    // workgroup -> (tile, column tile): the column tiles of one token tile share an XCD
    const int b = blockIdx.x;
    const int xcd = b % PF_XCD, i = b / PF_XCD;
    const int e = xcd + PF_XCD * (i / g.ntiles_n);
    const int jn = i % g.ntiles_n;
    if (e >= *g.n_tiles) return;
    const PfTile tl = g.tiles[e];
    // only the 32-row blocks that hold picks are loaded and staged
    // (the 2048-token layer, 36-83 picks per slot: 2.14 -> 2.09 ms)
    const int qa = (tl.rows + 31) >> 5;
    if (qa <= 1) pf_gemm_tile<MODE, NB, 1>(g, tl, jn, pf_lds);
    else if (qa == 2) pf_gemm_tile<MODE, NB, 2>(g, tl, jn, pf_lds);
    else if (qa == 3) pf_gemm_tile<MODE, NB, 3>(g, tl, jn, pf_lds);
    else pf_gemm_tile<MODE, NB, 4>(g, tl, jn, pf_lds);
}

// Stable grouping of the picks by slot, done by every workgroup of the
// decode gate/up kernel for itself (batches of at most DEC_SORT_MAX picks):
// slot counts in LDS, their prefix sums give each slot's first tile and first
// sorted position (slots ascending, DEC_MT picks per tile, the same list the
// separate sort writes); the workgroup's tile e then takes the picks of its
// slot whose rank (pick order) falls in its chunk.  Fills *tl and the tile's
// picks at dec_lds + DEC_SORT_ROWS; the workgroups of column tile 0 also write
// the tile and its picks for the down projection, workgroup 0 the tile count.
// Returns false when e is past the last tile (the whole workgroup).
constexpr int DEC_SORT_MAX = 1024;      // picks
constexpr int DEC_SORT_ROWS = 4096;     // byte offset of the tile's picks in LDS (after S <= 1024 counts)
constexpr int DEC_SORT_INFO = DEC_SORT_ROWS + DEC_MT * 4;
constexpr int DEC_SORT_SCR = DEC_SORT_INFO + 64;

template <int NTH>
__device__ bool dec_sort_tile(const PfArgs& g, int e, int jn, unsigned char* lds, PfTile* tl) {
    int* cnt = reinterpret_cast<int*>(lds);
    int* rows_pick = reinterpret_cast<int*>(lds + DEC_SORT_ROWS);
    int* info = reinterpret_cast<int*>(lds + DEC_SORT_INFO);
    int* scr = reinterpret_cast<int*>(lds + DEC_SORT_SCR);
    const int tid = threadIdx.x, P = g.sort_P, S = g.sort_S;
    constexpr int PPT = DEC_SORT_MAX / NTH;  // picks per thread, in pick order
    for (int s = tid; s < S; s += NTH) cnt[s] = 0;
    __syncthreads();
    int sv[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int p = tid * PPT + j;
        const int s = p < P ? g.sort_slots[p] : -1;
        sv[j] = (s >= 0 && s < S) ? s : -1;
        if (sv[j] >= 0) atomicAdd(&cnt[sv[j]], 1);  // LDS integer counts: order-free
    }
    __syncthreads();
    const int spt = (S + NTH - 1) / NTH;  // slots per thread, ascending
    int my_nt = 0, my_np = 0;
    for (int j = 0; j < spt; ++j) {
        const int s = tid * spt + j;
        if (s < S) {
            my_np += cnt[s];
            my_nt += (cnt[s] + DEC_MT - 1) / DEC_MT;
        }
    }
    // tiles and picks scanned together: both are at most 1024 (16 bits each)
    int packed_tot;
    const int packed = moe::block_exclusive_scan((my_nt << 16) | my_np, scr, &packed_tot);
    const int n_tiles = packed_tot >> 16;
    int toff = packed >> 16, poff = packed & 0xffff;
    for (int j = 0; j < spt; ++j) {
        const int s = tid * spt + j;
        if (s >= S) break;
        const int c = cnt[s], nt = (c + DEC_MT - 1) / DEC_MT;
        if (e >= toff && e < toff + nt) {
            const int r0 = (e - toff) * DEC_MT;
            info[0] = s;
            info[1] = poff + r0;
            info[2] = min(DEC_MT, c - r0);
            info[3] = r0;
        }
        toff += nt;
        poff += c;
    }
    if (blockIdx.x == 0 && tid == 0) *g.n_tiles_out = n_tiles;
    __syncthreads();
    if (e >= n_tiles) return false;
    const int slot = info[0], p0 = info[1], rows = info[2], r0 = info[3];
    int f = 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) f += sv[j] == slot;
    int tot;
    int rk = moe::block_exclusive_scan(f, scr, &tot) - r0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        if (sv[j] == slot) {
            if (rk >= 0 && rk < rows) rows_pick[rk] = tid * PPT + j;
            ++rk;
        }
    }
    __syncthreads();
    if (jn == 0) {
        if (tid < rows) g.pair_out[p0 + tid] = rows_pick[tid];
        if (tid == 0) g.tiles_out[e] = PfTile{p0, rows, slot, 0};
    }
    *tl = PfTile{p0, rows, slot, 0};
    return true;
}

// Decode-shaped tile: DEC_MT = 32 token rows (a slot holds a few picks at
// decode batch sizes) x 32 * NW weight rows; wave w owns weight rows
// [32 w, 32 w + 32) and all 32 token rows, so every wave has MFMA work and
// the A tile is small.  Gate/up: weight block w holds gate rows of 16 h
// columns followed by the up rows of the same columns, so output column c <
// 16 (gate) and c + 16 (up) of one wave pair up through one lane exchange.
// The k-loop is the grouped GEMM's: two register sets ahead of two LDS
// buffers, XOR-swizzled 16-byte chunks.
//
// Q8 (W8A8 weights): the same tiles and pipeline on v_mfma_i32_32x32x32_i8,
// whose operands take 16 bytes per lane in the same places as the bf16 one
// (a k-step is then 128 int8 elements), with exact int32 accumulators.  The
// gate/up A operand is x's int8 codes (made with the pick sort); its epilogue
// dequantises (acc * s_x) * s_w in fp32, evaluates SwiGLU in double, stores h
// in fp32 (sorted order) and stores, per pick, the max |h| over its own 64 h
// columns (one plain store per pick and column tile: no atomics, nothing to
// clear).  The down kernel quantises h itself: its prologue takes each pick's
// max over those column tiles (scale max / 127, 1 for a zero row), and the A
// operand is fetched as fp32 h and turned into int8 codes (round half to
// even, clamp 127) when it is stored to LDS; its epilogue is w * ((acc *
// s_h) * s_w).  The first k-steps' loads go out before the prologues, which
// only wait for small reads.  (Quantising x in the gate/up kernel as well,
// with the picks sorted there too, was slower: the sort's latency is exposed
// in every workgroup, which cannot fetch a weight before it knows its slot.)  This is the arithmetic of the row-streaming
// W8A8 kernels and of k_quant_rows, so the results match them.
template <int MODE, int NW, int NR, bool Q8 = false>
__global__ void __launch_bounds__(64 * NW) k_dec_gemm(PfArgs g) {
    constexpr int NTH = 64 * NW;
    constexpr int WR = 32 * NW;                  // weight rows per tile
    constexpr int ESZ = Q8 ? 1 : 2;               // bytes per operand element
    constexpr int A_BYTES = DEC_MT * PF_ROWB;     // 4 KiB per k-step
    constexpr int B_BYTES = WR * PF_ROWB;
    constexpr int NA = DEC_MT * 8 / NTH;          // A chunks per thread and k-step
    constexpr int NBU = WR * 8 / NTH;             // B chunks per thread and k-step (4)
    // the down kernel's int8 A operand is fetched as fp32 h and quantised on the way to LDS: four 16-byte
    // pieces per 16-byte chunk of codes
    constexpr bool AQ = Q8 && MODE == PF_DOWN;
    constexpr int APC = AQ ? 4 : 1;
    static_assert(NA >= 1 && NBU >= 1, "tile shape");
    extern __shared__ __attribute__((aligned(16))) unsigned char dec_lds[];
    __shared__ float q_row[DEC_MT];               // Q8: per token row, s_x (gate/up) or s_h (down)
    __shared__ float q_max[NW][DEC_MT];           // Q8 gate/up: per wave and token row, the max |h|
    const int b = blockIdx.x;
    const int xcd = b % PF_XCD, i = b / PF_XCD;
    const int e = xcd + PF_XCD * (i / g.ntiles_n);
    const int jn = i % g.ntiles_n;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    PfTile tl;
    const bool fused = MODE == PF_GU && g.sort_slots != nullptr;
    if (fused) {
        if (!dec_sort_tile<NTH>(g, e, jn, dec_lds, &tl)) return;
    } else {
        if (e >= *g.n_tiles) return;
        tl = g.tiles[e];
    }
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    const size_t row_bytes = (size_t)g.K * ESZ;

    const unsigned char* arow[NA];
    int aso[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        const int u = q * NTH + tid, r = u >> 3, ch = u & 7;
        const int rr = min(r, tl.rows - 1);  // rows past the picks repeat the last one (dropped)
        int idx;
        if constexpr (MODE == PF_GU)
            idx = (fused ? reinterpret_cast<const int32_t*>(dec_lds + DEC_SORT_ROWS)[rr] : g.pair_list[tl.p0 + rr]) /
                  g.k;
        else idx = tl.p0 + rr;
        arow[q] = g.act + (size_t)idx * row_bytes * APC + ch * 16 * APC;
        aso[q] = r * PF_ROWB + ((ch ^ swz(r)) * 16);
    }
    const unsigned char* brow[NBU];
    int bso[NBU];
#pragma unroll
    for (int q = 0; q < NBU; ++q) {
        const int u = q * NTH + tid, r = u >> 3, ch = u & 7;
        int64_t plane;
        int wr;
        if constexpr (MODE == PF_GU) {
            const int blk = r >> 5, c = r & 31;
            plane = c < 16 ? g.w0 : g.w1;
            wr = jn * (16 * NW) + blk * 16 + (c & 15);
        } else {
            plane = g.w0;
            wr = jn * WR + r;
        }
        brow[q] = slab + plane + (size_t)wr * row_bytes + ch * 16;
        bso[q] = r * PF_ROWB + ((ch ^ swz(r)) * 16);
    }
    const int khalf = lane >> 5, ar = lane & 31, br = wv * 32 + (lane & 31);
    int a_off[4], b_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        a_off[ks] = ar * PF_ROWB + (((ks * 2 + khalf) ^ swz(ar)) * 16);
        b_off[ks] = br * PF_ROWB + (((ks * 2 + khalf) ^ swz(br)) * 16);
    }
    using AccV = typename std::conditional<Q8, i32x16, f32x16>::type;
    AccV acc;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] = 0;

    const int nk = (int)(row_bytes / PF_ROWB);
    v4u ra[NR][NA * APC], rb[NR][NBU];
    float ascale[NA];  // Q8: the scale of each A chunk's token row
    const int rot = k_rot(nk);  // each workgroup walks k from its own starting step
    auto fetch = [&](v4u (&a)[NA * APC], v4u (&w)[NBU], int kt) {
        const int kr = kt + rot;
        const size_t ko = (size_t)(kr >= nk ? kr - nk : kr) * PF_ROWB;
#pragma unroll
        for (int q = 0; q < NA; ++q)
#pragma unroll
            for (int c = 0; c < APC; ++c) a[q * APC + c] = ld16(arow[q] + ko * APC + 16 * c);
#pragma unroll
        for (int q = 0; q < NBU; ++q) w[q] = ld16_nt(brow[q] + ko);
    };
    auto stash = [&](const v4u (&a)[NA * APC], const v4u (&w)[NBU], int buf) {
        unsigned char* A = dec_lds + buf * (A_BYTES + B_BYTES);
        unsigned char* B = A + A_BYTES;
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            if constexpr (AQ) {
                // 16 fp32 h values -> 16 int8 codes: rint(v / s), clamped to +-127
                uint32_t packed[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t word = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = __uint_as_float(a[q * APC + c][e]);
                        const float cd = fminf(fmaxf(rintf(v / ascale[q]), -127.0f), 127.0f);
                        word |= ((uint32_t)(int)cd & 0xFFu) << (8 * e);
                    }
                    packed[c] = word;
                }
                *reinterpret_cast<v4u*>(A + aso[q]) = v4u{packed[0], packed[1], packed[2], packed[3]};
            } else {
                *reinterpret_cast<v4u*>(A + aso[q]) = a[q];
            }
        }
#pragma unroll
        for (int q = 0; q < NBU; ++q) *reinterpret_cast<v4u*>(B + bso[q]) = w[q];
    };
    auto compute = [&](int buf) {
        const unsigned char* A = dec_lds + buf * (A_BYTES + B_BYTES);
        const unsigned char* B = A + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const v4u a16 = *reinterpret_cast<const v4u*>(A + a_off[ks]);
            const v4u b16 = *reinterpret_cast<const v4u*>(B + b_off[ks]);
            if constexpr (Q8)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a16),
                                                            __builtin_bit_cast(i32x4, b16), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16),
                                                              __builtin_bit_cast(bf16x8, b16), acc, 0, 0, 0);
        }
    };
    // NR register sets in a ring ahead of the two LDS buffers: step t is
    // fetched into set t % NR, stashed into buffer t % 2 one step before it
    // is computed.  The main loop runs U = lcm(2, NR) steps per pass with no
    // branch, so every wait on outstanding loads is exact; the last steps
    // (whose fetches would run past the end) are a guarded tail.
    constexpr int U = NR % 2 == 0 ? NR : 2 * NR;
#pragma unroll
    for (int r = 0; r < NR; ++r)
        if (r < nk) fetch(ra[r], rb[r], r);
    if constexpr (Q8) {
        // the token rows' scales, while the first k-steps are in flight
        if constexpr (MODE == PF_GU) {
            // each token row's activation scale (made with x's codes)
            if (tid < DEC_MT && tid < tl.rows) {
                const int pk = fused ? reinterpret_cast<const int32_t*>(dec_lds + DEC_SORT_ROWS)[tid]
                                     : g.pair_list[tl.p0 + tid];
                q_row[tid] = g.xscale[pk / g.k];
            }
        } else {
            // h's per-row scale from the gate/up column tiles' maxima of |h|
            if (tid < DEC_MT && tid < tl.rows) {
                float mx = 0.0f;
                for (int j = 0; j < g.K / 64; ++j) mx = fmaxf(mx, g.hmax[(size_t)j * g.hstride + tl.p0 + tid]);
                q_row[tid] = mx > 0.0f ? mx / 127.0f : 1.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NA; ++q) ascale[q] = q_row[min((q * NTH + tid) >> 3, tl.rows - 1)];
    }
    if (fused) __syncthreads();  // the sort's LDS is the first k-step's buffer
    stash(ra[0], rb[0], 0);
    lds_barrier();
    auto step = [&](int j, int t, bool tail) {  // j = t % U, static in every caller
        if (!tail || t + NR < nk) fetch(ra[j % NR], rb[j % NR], t + NR);  // set j % NR went to LDS last step
        compute(j % 2);
        if (!tail || t + 1 < nk) stash(ra[(j + 1) % NR], rb[(j + 1) % NR], (j + 1) % 2);
        lds_barrier();
    };
    int kt = 0;
    for (; kt + U + NR <= nk; kt += U) {  // every fetch of these steps is in range
#pragma unroll
        for (int j = 0; j < U; ++j) step(j, kt + j, false);
    }
#pragma unroll
    for (int j = 0; j < U + NR; ++j)
        if (kt + j < nk) step(j % U, kt + j, true);

    // accumulator element x of lane l: column l % 32 of this wave's block, row (x/4)*8 + (l/32)*4 + x%4
    const int col = lane & 31;
    if constexpr (MODE == PF_GU) {
        const int n = jn * (16 * NW) + wv * 16 + (col & 15);  // the h column (gate row and up row) of this lane
        float sg = 0.0f, su = 0.0f;
        if constexpr (Q8) {
            sg = reinterpret_cast<const float*>(slab + g.s0)[n];
            su = reinterpret_cast<const float*>(slab + g.s1)[n];
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const auto up = __shfl_xor(acc[x], 16, 64);  // every lane takes part
            const int r = (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if constexpr (Q8) {
                float hv = 0.0f;
                if (r < tl.rows && col < 16) {
                    const float sx = q_row[r];
                    const float gv = ((float)acc[x] * sx) * sg;
                    const float uv = ((float)up * sx) * su;
                    hv = (float)(((double)gv / (1.0 + exp(-(double)gv))) * (double)uv);
                    reinterpret_cast<float*>(g.out)[(size_t)(tl.p0 + r) * g.N + n] = hv;
                }
                // max |h| of row r over this wave's 16 h columns (lanes col 0..15 of the half-wave; the up
                // lanes hold 0)
                float mx = fabsf(hv);
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
                if (col == 0) q_max[wv][r] = mx;
            } else if (r < tl.rows && col < 16) {
                const float gv = acc[x];
                const float hv = gv / (1.0f + expf(-gv)) * up;
                reinterpret_cast<uint16_t*>(g.out)[(size_t)(tl.p0 + r) * g.N + n] = moe::f32_to_bf16(hv);
            }
        }
        if constexpr (Q8) {  // this column tile's max |h| per pick, over its 16 * NW h columns
            __syncthreads();
            if (tid < tl.rows) {
                float mx = q_max[0][tid];
#pragma unroll
                for (int w = 1; w < NW; ++w) mx = fmaxf(mx, q_max[w][tid]);
                g.hmax[(size_t)jn * g.hstride + tl.p0 + tid] = mx;
            }
        }
    } else {
        float* part = reinterpret_cast<float*>(g.out);
        const int m = jn * WR + wv * 32 + col;  // output column (down row) of this lane
        const float sd = Q8 ? reinterpret_cast<const float*>(slab + g.s0)[m] : 1.0f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            const int pk = g.pair_list[tl.p0 + r];
            if constexpr (Q8) part[(size_t)pk * g.N + m] = g.wts[pk] * (((float)acc[x] * q_row[r]) * sd);
            else part[(size_t)pk * g.N + m] = g.wts[pk] * acc[x];
        }
    }
}

// Large token groups (hundreds of picks per slot): tiles of 256 token rows x
// 256 weight rows, so every weight row is read once per 256 tokens.
constexpr int PB_MT = 256;  // token rows per tile
constexpr int PB_NT = 256;  // weight rows per tile

// The tiles are multiplied with the operands carried straight from memory
// into LDS: four waves, wave (wr, wc) computing token rows [128 wr, 128 wr +
// 128) against weight rows [128 wc, 128 wc + 128) as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs), so one LDS operand read
// feeds four MFMAs.  A k-step covers 64 k: whole 128-byte lines of every row
// (row pieces of half a line halve the rate of the loads).  The 160 KiB of
// LDS hold two k-steps of the token operand and three of the weight operand
// (the one that misses in L2): the weight loads of step t + 2 go out while
// the first half of step t is multiplied, the token loads of t + 2 while its
// last quarter is, each spread over the MFMAs.  The loads write LDS in lane
// order (lane l of a load fills bytes 16 l of its 1 KiB), so the swizzle that
// keeps the MFMA operand reads free of bank conflicts is applied on the memory
// side: LDS chunk s of row r holds the row's 16-byte chunk s ^ swz(r).
constexpr int PW_THREADS = 256;
constexpr int PW_OPB = 256 * PF_ROWB;     // 32 KiB: one operand of one k-step
constexpr int PW_NA = 2, PW_NB = 3;       // k-steps held per operand
constexpr int PW_LDS = (PW_NA + PW_NB) * PW_OPB;
constexpr int PW_LD = PW_OPB / 1024 / 4;  // 1 KiB loads per operand, wave and k-step
static_assert(PW_LDS <= 160 * 1024, "LDS of one CU");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt for at most N outstanding vector memory operations and no
// outstanding LDS reads (exp untouched)
template <int N>
__device__ __forceinline__ void pw_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// workgroup barrier of the load ring.  The waits before it are explicit
// (pw_wait_vm: this wave's buffer loads of the next step are in LDS and its
// LDS reads are done), so it is a bare s_barrier: a fence here would make the
// compiler wait for every buffer load in flight, the ones of later steps too.
// The memory clobber keeps LDS reads and loads on their side of it.
__device__ __forceinline__ void pw_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pw_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <int MODE>
__global__ void __launch_bounds__(PW_THREADS) k_pf_wide(PfArgs g) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[PW_LDS];
    // workgroup -> (tile, column tile): each XCD takes a contiguous run of the
    // tiles (the tiles of one slot are adjacent in the list) and walks them
    // with the column tile fastest, so the token tiles of a slot read each
    // weight tile at about the same time from the XCD's L2, and the column
    // tiles of a token tile share its activations there
    const int b = blockIdx.x;
    const int xcd = b % PF_XCD, i = b / PF_XCD;
    const int nt = *g.n_tiles;
    const int per_xcd = (nt + PF_XCD - 1) / PF_XCD;
    const int local = i / g.ntiles_n;
    const int e = xcd * per_xcd + local;
    const int jn = i % g.ntiles_n;
    if (local >= per_xcd || e >= nt) return;
    const PfTile tl = g.tiles[e];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: buffer resources and LDS bases in SGPRs
    const int wr = wv >> 1, wc = wv & 1;
    const int row_bytes = g.K * 2;

    // load j of wave wv fills LDS rows 64 wv + 8 j + lane / 8 of an operand
    uint32_t voff_a[PW_LD], voff_b[PW_LD];
#pragma unroll
    for (int j = 0; j < PW_LD; ++j) {
        const int r = wv * 64 + j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        const int pos = tl.p0 + min(r, tl.rows - 1);  // rows past the picks repeat the last one (dropped)
        int idx, w_row;
        if constexpr (MODE == PF_GU) {
            idx = g.pair_list[pos] / g.k;
            // weight rows of wave column c: gate rows of 64 h columns, then their up rows;
            // wave wv loads gate rows when wv is even, up rows when odd
            w_row = jn * 128 + (wv >> 1) * 64 + j * 8 + (lane >> 3);
        } else {
            idx = pos;
            w_row = jn * 256 + r;
        }
        voff_a[j] = (uint32_t)idx * (uint32_t)row_bytes + (uint32_t)(c * 16);
        voff_b[j] = (uint32_t)w_row * (uint32_t)row_bytes + (uint32_t)(c * 16);
    }
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    int64_t plane;
    if constexpr (MODE == PF_GU) plane = (wv & 1) ? g.w1 : g.w0;
    else plane = g.w0;
    // 32-bit buffer offsets: the host takes this kernel only for operands
    // under 2 GiB (moe_pf_big)
    const __amdgpu_buffer_rsrc_t ra = pw_rsrc(g.act, 0x7fffffff);
    const __amdgpu_buffer_rsrc_t rb = pw_rsrc(slab + plane, g.N * row_bytes);

    // the k walk starts at a step of the slot's own: the workgroups that share
    // a token tile (all column tiles) or a weight tile (all token tiles of the
    // slot) walk in step, so the second reader of a line finds it in L2
    const int nk = g.K / PF_KT;
    const int rot = (nk * PF_ROWB) % 4096 == 0 ? tl.slot % nk : 0;
    unsigned char* const lds_a = lds;
    unsigned char* const lds_b = lds + PW_NA * PW_OPB;
    auto koff = [&](int kt) {
        const int kr = kt + rot;
        return (kr >= nk ? kr - nk : kr) * PF_ROWB;
    };
    // load j of step kt of the token (A) or weight (B) operand
    auto load_a = [&](int kt, int j) {
        unsigned char* base = lds_a + (kt % PW_NA) * PW_OPB + wv * (PW_LD * 1024);
        const int so = koff(kt);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + j * 1024), 16, voff_a[j], so, 0, 0);
    };
    auto load_b = [&](int kt, int j) {
        unsigned char* base = lds_b + (kt % PW_NB) * PW_OPB + wv * (PW_LD * 1024);
        const int so = koff(kt);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(base + j * 1024), 16, voff_b[j], so, 0, 0);
    };

    // operand rows of a lane: (128 wr or 128 wc) + 32 blk + lane % 32, whose
    // swizzle is swz(lane % 32) ^ 4 for odd blocks
    const int l32 = lane & 31, kh = lane >> 5, f0 = swz(l32);
    const int a_lane = (wr * 128 + l32) * PF_ROWB, b_lane = (wc * 128 + l32) * PF_ROWB;
    f32x16 acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mb][nb][x] = 0.0f;
    // operands of quarter ks (16 k) of step t
    auto read = [&](int t, int ks, bf16x8* av, bf16x8* bv) {
        const unsigned char* A = lds_a + (t % PW_NA) * PW_OPB;
        const unsigned char* B = lds_b + (t % PW_NB) * PW_OPB;
        const int c = ks * 2 + kh;
        const int co0 = (c ^ f0) * 16, co1 = (c ^ f0 ^ 4) * 16;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            av[mb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const v4u*>(A + a_lane + mb * 32 * PF_ROWB + ((mb & 1) ? co1 : co0)));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            bv[nb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const v4u*>(B + b_lane + nb * 32 * PF_ROWB + ((nb & 1) ? co1 : co0)));
    };
    // the sixteen MFMAs of a quarter, with buffer loads of step kt after each
    // four of them (the loads go out spread over the MFMAs: issued in one burst
    // they fill the address queue and hold up the MFMA issue behind them):
    // LD_NONE, the weight loads 0..3 or 4..7 (one per four MFMAs), or the token
    // loads (two per four MFMAs)
    enum { LD_NONE, LD_B_LO, LD_B_HI, LD_A };
    auto mfma = [&](const bf16x8* av, const bf16x8* bv, int what, int kt) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (what == LD_B_LO) load_b(kt, mb);
            else if (what == LD_B_HI) load_b(kt, 4 + mb);
            else if (what == LD_A) {
                load_a(kt, 2 * mb);
                load_a(kt, 2 * mb + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    bf16x8 a0[4], b0[4], a1[4], b1[4];
    // quarters 0..2 of step t, the weight loads of step kb (if kb >= 0) spread
    // over quarters 0 and 1; the reads of the next quarter go out before the
    // MFMAs of this one
    auto body = [&](int t, int kb) {
        read(t, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma(a0, b0, kb >= 0 ? LD_B_LO : LD_NONE, kb);
        read(t, 2, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma(a1, b1, kb >= 0 ? LD_B_HI : LD_NONE, kb);
        read(t, 3, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma(a0, b0, LD_NONE, 0);
    };

    // Step t: quarters 0..2 (with the weight loads of t + 2); wait for this
    // wave's loads of t + 1 (only the weight loads of t + 2 may be
    // outstanding) and barrier, after which every wave's loads of t + 1 are in
    // LDS and every wave is done reading t, whose token buffer takes the loads
    // of t + 2; read quarter 0 of t + 1 and multiply quarter 3 of t with those
    // loads spread over it.  The weight buffer of t + 2 was last read at step
    // t - 1.  Waves past the tile's rows multiply the repeated last row
    // (dropped), so the loops have no branches and the accumulators stay in
    // AGPRs.  nk >= 2.
#pragma unroll
    for (int j = 0; j < PW_LD; ++j) load_a(0, j);
#pragma unroll
    for (int j = 0; j < PW_LD; ++j) load_b(0, j);
#pragma unroll
    for (int j = 0; j < PW_LD; ++j) load_a(1, j);
#pragma unroll
    for (int j = 0; j < PW_LD; ++j) load_b(1, j);
    pw_wait_vm<2 * PW_LD>();
    pw_barrier();
    read(0, 0, a0, b0);
    int t = 0;
    for (; t + 2 < nk; ++t) {
        body(t, t + 2);
        pw_wait_vm<PW_LD>();
        pw_barrier();
        read(t + 1, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma(a1, b1, LD_A, t + 2);
    }
    // t = nk - 2
    body(t, -1);
    pw_wait_vm<0>();
    pw_barrier();
    read(t + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mfma(a1, b1, LD_NONE, 0);
    ++t;
    // t = nk - 1
    body(t, -1);
    mfma(a1, b1, LD_NONE, 0);

    // the pick and routing weight of each tile row, staged in LDS once the
    // loop is done with it (the down projection scales its rows by them)
    int32_t* row_pick = reinterpret_cast<int32_t*>(lds);
    float* row_wt = reinterpret_cast<float*>(lds + 1024);
    if constexpr (MODE == PF_DOWN) {
        const int pk = g.pair_list[tl.p0 + min(tid, tl.rows - 1)];
        const float wt = g.wts[pk];
        __syncthreads();
        row_pick[tid] = pk;
        row_wt[tid] = wt;
        __syncthreads();
    }

    if (wr * 128 >= tl.rows) return;
    const int col = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = wr * 128 + mb * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            if constexpr (MODE == PF_GU) {
                uint16_t* h = reinterpret_cast<uint16_t*>(g.out);
                const size_t hrow = (size_t)(tl.p0 + r) * g.N + jn * 128 + wc * 64;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float gv = acc[mb][half][x], uv = acc[mb][2 + half][x];
                    // silu with the hardware exp and reciprocal: the result is rounded to bf16
                    const float sg = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
                    h[hrow + half * 32 + col] = moe::f32_to_bf16(sg * uv);
                }
            } else {
                uint16_t* part = reinterpret_cast<uint16_t*>(g.out);  // bf16 partials, as k_pf_gemm
                const int pk = row_pick[r];
                const float wt = row_wt[r];
                uint16_t* prow = part + (size_t)pk * g.N + jn * 256 + wc * 128;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) prow[nb * 32 + col] = moe::f32_to_bf16(wt * acc[mb][nb][x]);
            }
        }
    }
}

int pb_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
              const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
              int max_tiles, void* hbuf, float* part, hipStream_t st) {
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k,
              I / (PB_NT / 2)};
    hipLaunchKernelGGL((k_pf_wide<PF_GU>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)), dim3(PW_THREADS), 0,
                       st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/large_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k, H / PB_NT};
    hipLaunchKernelGGL((k_pf_wide<PF_DOWN>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)), dim3(PW_THREADS),
                       0, st, dn);
    return moe_check_launch("moe_ffn_slots/large_down");
}

template <int NW, bool Q8>
int dec_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
               const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
               int max_tiles, void* hbuf, float* part, hipStream_t st, const int32_t* sort_slots, int P, int S,
               const float* xscale, float* hmax) {
    const int lds = 2 * (DEC_MT + 32 * NW) * PF_ROWB;
    static_assert(DEC_SORT_SCR + 64 <= 2 * (DEC_MT + 32 * DEC_NW) * PF_ROWB, "the sort fits the kernel's LDS");
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k, I / (16 * NW)};
    if (sort_slots) {  // the gate/up workgroups sort the picks (and write the lists the down kernel reads)
        gu.sort_slots = sort_slots;
        gu.sort_P = P;
        gu.sort_S = S;
        gu.pair_out = const_cast<int32_t*>(pair_list);
        gu.tiles_out = const_cast<PfTile*>(tiles);
        gu.n_tiles_out = const_cast<int32_t*>(n_tiles);
    }
    if (Q8) {
        gu.s0 = lay.s[0];
        gu.s1 = lay.s[1];
        gu.xscale = xscale;
        gu.hmax = hmax;
        gu.hstride = P;
    }
    hipLaunchKernelGGL((k_dec_gemm<PF_GU, NW, DEC_NR_GU, Q8>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)),
                       dim3(64 * NW), lds, st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/decode_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k,
              H / (32 * NW)};
    if (Q8) {
        dn.s0 = lay.s[2];
        dn.hmax = hmax;
        dn.hstride = P;
    }
    hipLaunchKernelGGL((k_dec_gemm<PF_DOWN, NW, DEC_NR_DN, Q8>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)),
                       dim3(64 * NW), lds, st, dn);
    return moe_check_launch("moe_ffn_slots/decode_down");
}

// NBG / NBD: 32-row weight blocks per wave of the gate/up and down GEMMs.
template <int NBG, int NBD>
int pf_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
              const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
              int max_tiles, void* hbuf, float* part, hipStream_t st) {
    // 64 KiB of LDS at NB = 4, 96 KiB at NB = 8: allowed once per device (under a lock, so
    // threads that launch on several devices at once each see it done for theirs)
    static std::mutex mu;
    static uint64_t done = 0;  // bit d: set for device d
    const int lds_g = pf_lds_bytes(NBG), lds_d = pf_lds_bytes(NBD);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return moe_fail(MOE_E_HIP, "moe_ffn_slots: no current device (or device %d beyond 63)", dev);
    }
    {
        std::lock_guard<std::mutex> lk(mu);
        if (!(done >> dev & 1)) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_gemm<PF_GU, NBG>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds_g) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_gemm<PF_DOWN, NBD>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds_d) != hipSuccess) {
                (void)hipGetLastError();
                return moe_fail(MOE_E_HIP, "moe_ffn_slots: cannot allow %d / %d bytes of LDS for the prefill kernels",
                                lds_g, lds_d);
            }
            done |= 1ull << dev;
        }
    }
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k, I / (NBG * 16)};
    hipLaunchKernelGGL((k_pf_gemm<PF_GU, NBG>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)),
                       dim3(PF_THREADS), lds_g, st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/prefill_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k,
              H / (NBD * 32)};
    hipLaunchKernelGGL((k_pf_gemm<PF_DOWN, NBD>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)),
                       dim3(PF_THREADS), lds_d, st, dn);
    return moe_check_launch("moe_ffn_slots/prefill_down");
}

}  // namespace

bool moe_pf_supported(int w_type, int H, int I) {
    // column tiles of 64 h columns / 128 output rows; contraction in 128-byte steps (pairs of them for bf16)
    return (w_type == MOE_W_BF16 || w_type == MOE_W_W8A8) && H % 128 == 0 && I % 128 == 0;
}

int moe_pf_tile_rows(int T, int k) { return T * k < PF_BIG_P ? DEC_MT : PF_MT; }

bool moe_pf_big(int T, int k, int S, int H, int I) {
    // hundreds of picks per slot on average, and whole 256-row / 128-column tiles
    const int P = T * k;
    // the buffer loads address each operand with 31-bit offsets
    const bool fits = (int64_t)T * H * 2 < INT32_MAX && (int64_t)P * I * 2 < INT32_MAX &&
                      (int64_t)H * I * 2 < INT32_MAX;
    return fits && P >= PF_BIG_P && P / (S > 0 ? S : 1) >= PB_BIG_ROWS && H % PB_NT == 0 && I % 128 == 0 &&
           I >= 256;  // at least four 64-k steps in either contraction
}

int moe_pf_tile_rows(int T, int k, int S, int H, int I) {
    return moe_pf_big(T, k, S, H, I) ? PB_MT : moe_pf_tile_rows(T, k);
}

int moe_pf_tile_rows_for(int w_type, int T, int k, int S, int H, int I) {
    return w_type == MOE_W_W8A8 ? DEC_MT : moe_pf_tile_rows(T, k, S, H, I);
}

namespace {
// Bound on the tiles of `rows` picks the sort writes for P picks over S
// slots: each of the at most min(S, P) slots with picks adds at most one
// partial tile to its P_s / rows whole ones.
int pf_grid_tiles(int P, int S, int rows) { return (S < P ? S : P) + P / rows + 1; }
}  // namespace

int moe_pf_max_tiles(int T, int k, int S) {
    const int P = T * k;
    // bounds the sum over slots of ceil(n_s / rows) for every tile height in use (32 rows and up)
    return (S < P ? S : P) + P / DEC_MT + 1;
}

size_t moe_pf_tiles_bytes(int T, int k, int S) { return (size_t)moe_pf_max_tiles(T, k, S) * sizeof(PfTile) + 16; }

bool moe_pf_part_bf16(int w_type, int T, int k) { return w_type == MOE_W_BF16 && T * k >= PF_BIG_P; }

bool moe_pf_fused_sort(int T, int k) {
    const int P = T * k;
    return P < PF_BIG_P && P <= DEC_SORT_MAX;
}

int moe_pf_run(const void* x, const float* w, int T, int k, const void* slot_store, size_t slab_bytes, int S, int H,
               int I, const moe_slab_layout_t& lay, const int32_t* pair_list, void* tiles_ws, void* hbuf, float* part,
               hipStream_t st, const int32_t* sort_slots, int w_type, const float* xscale, float* hmax) {
    const int P = T * k;
    const int max_tiles = moe_pf_max_tiles(T, k, S);
    const PfTile* tiles = reinterpret_cast<const PfTile*>(tiles_ws);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(reinterpret_cast<unsigned char*>(tiles_ws) +
                                                              (size_t)max_tiles * sizeof(PfTile));
    if (w_type == MOE_W_W8A8) {
        // int8 weights: decode-shaped tiles at every batch size (x given as int8 codes with per-token scales;
        // the sort wrote 32-row tiles, moe_pf_tile_rows_for)
        // (2 waves per workgroup, or 3 / 4 register sets in the ring: slower at 16 tokens of the 128-expert layer)
        return dec_launch<DEC_NW, true>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles,
                                        max_tiles, hbuf, part, st, sort_slots, P, S, xscale, hmax);
    }

    // decode-sized batches (a few picks per slot): 32-row token tiles; large groups: 256-row tiles
    if (sort_slots && !moe_pf_fused_sort(T, k)) return moe_fail(MOE_E_ARG, "moe_pf_run: no fused sort for %d picks", P);
    if (P < PF_BIG_P)
        return dec_launch<DEC_NW, false>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles,
                                         max_tiles, hbuf, part, st, sort_slots, P, S, nullptr, nullptr);
    // the grids of the prefill-shaped kernels cover the tiles the sort can
    // write at their own height (workgroups past the tile count only exit,
    // but each is still dispatched: at 16384 tokens of the 288-expert layer
    // the 32-row bound launched ~46,000 of them for ~6,900 tiles)
    if (moe_pf_big(T, k, S, H, I))
        return pb_launch(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles,
                         pf_grid_tiles(P, S, PB_MT), hbuf, part, st);
    const int grid_tiles = pf_grid_tiles(P, S, PF_MT);
    // down: eight 32-row weight blocks per wave where the output columns come
    // in 256s (fewer, longer workgroups: the 2048-token layer 2.06 -> 2.02 ms);
    // gate/up: four (64 KiB of LDS, two workgroups per CU: 2.13 -> 2.08 ms
    // against eight; two blocks: 2.35 ms)
    if (H % 256 == 0)
        return pf_launch<4, 8>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles, grid_tiles,
                               hbuf, part, st);
    return pf_launch<4, 4>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles, grid_tiles, hbuf,
                           part, st);
}

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
//                list of (slot, up to PF_MT consecutive picks) tiles
//   k_pf_gemm<GU>   [g | u] = X_s [W_g; W_u]^T per tile of 64 h columns,
//                   SwiGLU epilogue, h (bf16, RNE) stored in sorted-pick order
//   k_pf_gemm<DOWN> O = H_s W_d^T per tile of 128 output columns,
//                   part[pick] = w * O (fp32)
//   k_dec_gemm<GU|DOWN>  the same two GEMMs on decode-shaped tiles
//   k_reduce     y[t] = sum over resident picks in top-k order (decode path's)
//
// Prefill-sized batches (4096 picks and more): a workgroup owns PF_MT = 128
// token rows x NB * 32 weight rows (NB = 4) and walks K in steps of 64.
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

#include "common.hpp"
#include "prefill.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
__device__ __forceinline__ int k_rot(int nk) {
    return (nk * PF_ROWB) % 4096 == 0 ? (int)(blockIdx.x % (unsigned)nk) : 0;
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
    void* out;                   // GU: h [P][I] bf16 (sorted order); DOWN: part [P][H] fp32
    int K;                       // contraction length (GU: H, DOWN: I)
    int N;                       // output columns (GU: I, DOWN: H)
    int k;                       // top-k (GU: token = pick / k)
    int ntiles_n;                // column tiles per token tile
};

__device__ __forceinline__ v4u ld16(const unsigned char* p) { return *reinterpret_cast<const v4u*>(p); }
__device__ __forceinline__ v4u ld16_nt(const unsigned char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}

template <int MODE, int NB>
__global__ void __launch_bounds__(PF_THREADS) k_pf_gemm(PfArgs g) {
    constexpr int HC = NB * 16;                          // gate/up: h columns per tile
    constexpr int B_BYTES = NB * 32 * PF_ROWB;           // B tile of one k-step
    extern __shared__ __attribute__((aligned(16))) unsigned char pf_lds[];
    // workgroup -> (tile, column tile): the column tiles of one token tile share an XCD
    const int b = blockIdx.x;
    const int xcd = b % PF_XCD, i = b / PF_XCD;
    const int e = xcd + PF_XCD * (i / g.ntiles_n);
    const int jn = i % g.ntiles_n;
    if (e >= *g.n_tiles) return;
    const PfTile tl = g.tiles[e];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    const size_t row_bytes = (size_t)g.K * 2;

    // this thread's 4 A rows and NB B rows (row = q * 32 + tid / 8, chunk tid % 8)
    const int lrow = tid >> 3, chunk = tid & 7;
    const unsigned char* arow[4];
    const unsigned char* brow[NB];
    int soff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = q * 32 + lrow;
        // rows past the tile's picks repeat its last row (a line the wave already reads; results dropped)
        const int pos = tl.p0 + min(r, tl.rows - 1);
        int arow_idx;
        if constexpr (MODE == PF_GU) arow_idx = g.pair_list[pos] / g.k;   // token of the pick
        else arow_idx = pos;                                             // h row in sorted order
        arow[q] = g.act + (size_t)arow_idx * row_bytes + chunk * 16;
        soff[q] = r * PF_ROWB + ((chunk ^ swz(r)) * 16);
        if (q < NB) {
            int wr;
            int64_t plane;
            if constexpr (MODE == PF_GU) {  // rows 0..HC-1 gate, HC..2HC-1 up, of h columns jn*HC ..
                plane = r < HC ? g.w0 : g.w1;
                wr = jn * HC + (r < HC ? r : r - HC);
            } else {
                plane = g.w0;
                wr = jn * (NB * 32) + r;
            }
            brow[q < NB ? q : 0] = slab + plane + (size_t)wr * row_bytes + chunk * 16;
        }
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
    v4u ra[2][4], rb[2][NB];
    // each workgroup walks k from its own starting step (see k_rot)
    const int rot = k_rot(nk);
    auto fetch = [&](v4u (&a)[4], v4u (&w)[NB], int kt) {
        const int kr = kt + rot;
        const size_t ko = (size_t)(kr >= nk ? kr - nk : kr) * PF_ROWB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a[q] = ld16(arow[q] + ko);
            if (q < NB) w[q < NB ? q : 0] = ld16_nt(brow[q < NB ? q : 0] + ko);
        }
    };
    auto stash = [&](const v4u (&a)[4], const v4u (&w)[NB], int buf) {
        unsigned char* A = pf_lds + buf * (PF_TILE_BYTES + B_BYTES);
        unsigned char* B = A + PF_TILE_BYTES;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<v4u*>(A + soff[q]) = a[q];
            if (q < NB) *reinterpret_cast<v4u*>(B + soff[q]) = w[q < NB ? q : 0];
        }
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
    __syncthreads();
    for (int kt = 0; kt + 2 < nk; kt += 2) {
        fetch(ra[0], rb[0], kt + 2);  // buffer 0 holds step kt, registers 1 hold kt + 1
        compute(0);
        stash(ra[1], rb[1], 1);
        __syncthreads();
        fetch(ra[1], rb[1], kt + 3);  // buffer 1 holds kt + 1, registers 0 hold kt + 2
        compute(1);
        stash(ra[0], rb[0], 0);
        __syncthreads();
    }
    // last two steps: buffer 0 holds nk - 2, registers 1 hold nk - 1
    compute(0);
    stash(ra[1], rb[1], 1);
    __syncthreads();
    compute(1);

    if (!active_wave) return;
    // accumulator element x of lane l: column l % 32 of block nb, row (x/4)*8 + (l/32)*4 + x%4
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
                h[hrow + half * 32 + col] = moe::f32_to_bf16(hv);
            }
        }
    } else {
        float* part = reinterpret_cast<float*>(g.out);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = wv * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            const int pk = g.pair_list[tl.p0 + r];
            const float wt = g.wts[pk];
            float* prow = part + (size_t)pk * g.N + jn * (NB * 32);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) prow[nb * 32 + col] = wt * acc[nb][x];
        }
    }
}

// Decode-shaped tile: DEC_MT = 32 token rows (a slot holds a few picks at
// decode batch sizes) x 32 * NW weight rows; wave w owns weight rows
// [32 w, 32 w + 32) and all 32 token rows, so every wave has MFMA work and
// the A tile is small.  Gate/up: weight block w holds gate rows of 16 h
// columns followed by the up rows of the same columns, so output column c <
// 16 (gate) and c + 16 (up) of one wave pair up through one lane exchange.
// The k-loop is the grouped GEMM's: two register sets ahead of two LDS
// buffers, XOR-swizzled 16-byte chunks.
template <int MODE, int NW, int NR>
__global__ void __launch_bounds__(64 * NW) k_dec_gemm(PfArgs g) {
    constexpr int NTH = 64 * NW;
    constexpr int WR = 32 * NW;                  // weight rows per tile
    constexpr int A_BYTES = DEC_MT * PF_ROWB;     // 4 KiB per k-step
    constexpr int B_BYTES = WR * PF_ROWB;
    constexpr int NA = DEC_MT * 8 / NTH;          // A chunks per thread and k-step
    constexpr int NBU = WR * 8 / NTH;             // B chunks per thread and k-step (4)
    static_assert(NA >= 1 && NBU >= 1, "tile shape");
    extern __shared__ __attribute__((aligned(16))) unsigned char dec_lds[];
    const int b = blockIdx.x;
    const int xcd = b % PF_XCD, i = b / PF_XCD;
    const int e = xcd + PF_XCD * (i / g.ntiles_n);
    const int jn = i % g.ntiles_n;
    if (e >= *g.n_tiles) return;
    const PfTile tl = g.tiles[e];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    const size_t row_bytes = (size_t)g.K * 2;

    const unsigned char* arow[NA];
    int aso[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        const int u = q * NTH + tid, r = u >> 3, ch = u & 7;
        const int pos = tl.p0 + min(r, tl.rows - 1);  // rows past the picks repeat the last one (dropped)
        int idx;
        if constexpr (MODE == PF_GU) idx = g.pair_list[pos] / g.k;
        else idx = pos;
        arow[q] = g.act + (size_t)idx * row_bytes + ch * 16;
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
    f32x16 acc;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] = 0.0f;

    const int nk = g.K / PF_KT;
    v4u ra[NR][NA], rb[NR][NBU];
    const int rot = k_rot(nk);  // each workgroup walks k from its own starting step
    auto fetch = [&](v4u (&a)[NA], v4u (&w)[NBU], int kt) {
        const int kr = kt + rot;
        const size_t ko = (size_t)(kr >= nk ? kr - nk : kr) * PF_ROWB;
#pragma unroll
        for (int q = 0; q < NA; ++q) a[q] = ld16(arow[q] + ko);
#pragma unroll
        for (int q = 0; q < NBU; ++q) w[q] = ld16_nt(brow[q] + ko);
    };
    auto stash = [&](const v4u (&a)[NA], const v4u (&w)[NBU], int buf) {
        unsigned char* A = dec_lds + buf * (A_BYTES + B_BYTES);
        unsigned char* B = A + A_BYTES;
#pragma unroll
        for (int q = 0; q < NA; ++q) *reinterpret_cast<v4u*>(A + aso[q]) = a[q];
#pragma unroll
        for (int q = 0; q < NBU; ++q) *reinterpret_cast<v4u*>(B + bso[q]) = w[q];
    };
    auto compute = [&](int buf) {
        const unsigned char* A = dec_lds + buf * (A_BYTES + B_BYTES);
        const unsigned char* B = A + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(A + a_off[ks]));
            const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(B + b_off[ks]));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
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
    stash(ra[0], rb[0], 0);
    __syncthreads();
    auto step = [&](int j, int t, bool tail) {  // j = t % U, static in every caller
        if (!tail || t + NR < nk) fetch(ra[j % NR], rb[j % NR], t + NR);  // set j % NR went to LDS last step
        compute(j % 2);
        if (!tail || t + 1 < nk) stash(ra[(j + 1) % NR], rb[(j + 1) % NR], (j + 1) % 2);
        __syncthreads();
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
        uint16_t* h = reinterpret_cast<uint16_t*>(g.out);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const float up = __shfl_xor(acc[x], 16, 64);  // every lane takes part
            const int r = (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r < tl.rows && col < 16) {
                const float gv = acc[x];
                const float hv = gv / (1.0f + expf(-gv)) * up;
                h[(size_t)(tl.p0 + r) * g.N + jn * (16 * NW) + wv * 16 + col] = moe::f32_to_bf16(hv);
            }
        }
    } else {
        float* part = reinterpret_cast<float*>(g.out);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            const int pk = g.pair_list[tl.p0 + r];
            part[(size_t)pk * g.N + jn * WR + wv * 32 + col] = g.wts[pk] * acc[x];
        }
    }
}

// Large token groups (hundreds of picks per slot): 256 token rows x 256
// weight rows per workgroup of 8 waves, wave (wr, wc) computing token rows
// [64 wr, 64 wr + 64) against weight rows [128 wc, 128 wc + 128): 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16, so each LDS operand read feeds two or
// four MFMAs, and every weight row is read once per 256 tokens.  Gate/up:
// the 128 weight rows of a wave are 64 gate rows and the up rows of the same
// 64 h columns.  One register set of the next k-step is in flight while the
// current one is multiplied; two LDS buffers of 64 KiB.
constexpr int PB_THREADS = 512;
constexpr int PB_MT = 256;                           // token rows per tile
constexpr int PB_NT = 256;                           // weight rows per tile
constexpr int PB_A_BYTES = PB_MT * PF_ROWB;           // 32 KiB
constexpr int PB_B_BYTES = PB_NT * PF_ROWB;           // 32 KiB
constexpr int PB_LDS = 2 * (PB_A_BYTES + PB_B_BYTES);  // 128 KiB

template <int MODE>
__global__ void __launch_bounds__(PB_THREADS) k_pf_big(PfArgs g) {
    extern __shared__ __attribute__((aligned(16))) unsigned char pb_lds[];
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
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wr = wv >> 1, wc = wv & 1;
    const unsigned char* slab = g.slots + (size_t)tl.slot * g.slab_bytes;
    const size_t row_bytes = (size_t)g.K * 2;

    // this thread's 4 A and 4 B chunks of a k-step: row u / 8, chunk u % 8 for u = q * 512 + tid
    const unsigned char* arow[4];
    const unsigned char* brow[4];
    int soff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int u = q * PB_THREADS + tid, r = u >> 3, ch = u & 7;
        const int pos = tl.p0 + min(r, tl.rows - 1);  // rows past the picks repeat the last one (dropped)
        int idx;
        if constexpr (MODE == PF_GU) idx = g.pair_list[pos] / g.k;
        else idx = pos;
        arow[q] = g.act + (size_t)idx * row_bytes + ch * 16;
        soff[q] = r * PF_ROWB + ((ch ^ swz(r)) * 16);
        int64_t plane;
        int w_row;
        if constexpr (MODE == PF_GU) {
            const int half = r >> 7, rr = r & 127;
            plane = rr < 64 ? g.w0 : g.w1;
            w_row = jn * 128 + half * 64 + (rr & 63);
        } else {
            plane = g.w0;
            w_row = jn * PB_NT + r;
        }
        brow[q] = slab + plane + (size_t)w_row * row_bytes + ch * 16;
    }
    const int khalf = lane >> 5;
    int a_off[4][2], b_off[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int r = wr * 64 + mb * 32 + (lane & 31);
            a_off[ks][mb] = r * PF_ROWB + (((ks * 2 + khalf) ^ swz(r)) * 16);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int r = wc * 128 + nb * 32 + (lane & 31);
            b_off[ks][nb] = r * PF_ROWB + (((ks * 2 + khalf) ^ swz(r)) * 16);
        }
    }
    const bool active_wave = wr * 64 < tl.rows;
    f32x16 acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mb][nb][x] = 0.0f;

    const int nk = g.K / PF_KT;
    const int rot = k_rot(nk);
    v4u ra[4], rb[4];
    auto fetch = [&](int kt) {
        const int kr = kt + rot;
        const size_t ko = (size_t)(kr >= nk ? kr - nk : kr) * PF_ROWB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ra[q] = ld16(arow[q] + ko);
            rb[q] = ld16_nt(brow[q] + ko);
        }
    };
    auto stash = [&](int buf) {
        unsigned char* A = pb_lds + buf * (PB_A_BYTES + PB_B_BYTES);
        unsigned char* B = A + PB_A_BYTES;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<v4u*>(A + soff[q]) = ra[q];
            *reinterpret_cast<v4u*>(B + soff[q]) = rb[q];
        }
    };
    auto compute = [&](int buf) {
        if (!active_wave) return;
        const unsigned char* A = pb_lds + buf * (PB_A_BYTES + PB_B_BYTES);
        const unsigned char* B = A + PB_A_BYTES;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 av[2], bv[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                av[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(A + a_off[ks][mb]));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                bv[nb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u*>(B + b_off[ks][nb]));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
    };
    // step t: the loads of t + 1 are in flight while t is multiplied out of buffer t % 2
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt + 2 <= nk; kt += 2) {  // nk is even
        if (kt + 1 < nk) fetch(kt + 1);
        compute(0);
        stash(1);
        __syncthreads();
        if (kt + 2 < nk) fetch(kt + 2);
        compute(1);
        if (kt + 2 < nk) stash(0);
        __syncthreads();
    }

    if (!active_wave) return;
    const int col = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = wr * 64 + mb * 32 + (x >> 2) * 8 + (lane >> 5) * 4 + (x & 3);
            if (r >= tl.rows) continue;
            if constexpr (MODE == PF_GU) {
                uint16_t* h = reinterpret_cast<uint16_t*>(g.out);
                const size_t hrow = (size_t)(tl.p0 + r) * g.N + jn * 128 + wc * 64;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float gv = acc[mb][half][x], uv = acc[mb][2 + half][x];
                    h[hrow + half * 32 + col] = moe::f32_to_bf16(gv / (1.0f + expf(-gv)) * uv);
                }
            } else {
                float* part = reinterpret_cast<float*>(g.out);
                const int pk = g.pair_list[tl.p0 + r];
                const float wt = g.wts[pk];
                float* prow = part + (size_t)pk * g.N + jn * PB_NT + wc * 128;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) prow[nb * 32 + col] = wt * acc[mb][nb][x];
            }
        }
    }
}

int pb_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
              const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
              int max_tiles, void* hbuf, float* part, hipStream_t st) {
    static bool lds_set = false;
    if (!lds_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_big<PF_GU>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, PB_LDS) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_big<PF_DOWN>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, PB_LDS) != hipSuccess) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_HIP, "moe_ffn_slots: cannot allow %d bytes of LDS for the large-group kernels",
                            PB_LDS);
        }
        lds_set = true;
    }
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k, I / 128};
    hipLaunchKernelGGL((k_pf_big<PF_GU>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)), dim3(PB_THREADS),
                       PB_LDS, st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/large_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k, H / PB_NT};
    hipLaunchKernelGGL((k_pf_big<PF_DOWN>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)), dim3(PB_THREADS),
                       PB_LDS, st, dn);
    return moe_check_launch("moe_ffn_slots/large_down");
}

template <int NW>
int dec_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
               const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
               int max_tiles, void* hbuf, float* part, hipStream_t st) {
    const int lds = 2 * (DEC_MT + 32 * NW) * PF_ROWB;
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k, I / (16 * NW)};
    hipLaunchKernelGGL((k_dec_gemm<PF_GU, NW, DEC_NR_GU>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)),
                       dim3(64 * NW), lds, st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/decode_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k,
              H / (32 * NW)};
    hipLaunchKernelGGL((k_dec_gemm<PF_DOWN, NW, DEC_NR_DN>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)),
                       dim3(64 * NW), lds, st, dn);
    return moe_check_launch("moe_ffn_slots/decode_down");
}

template <int NB>
int pf_launch(const void* x, const float* w, int k, const void* slot_store, size_t slab_bytes, int H, int I,
              const moe_slab_layout_t& lay, const int32_t* pair_list, const PfTile* tiles, const int32_t* n_tiles,
              int max_tiles, void* hbuf, float* part, hipStream_t st) {
    static bool lds_set = false;  // once per process: the kernels need more than 64 KiB of LDS only at NB = 4
    const int lds = pf_lds_bytes(NB);
    if (!lds_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_gemm<PF_GU, NB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf_gemm<PF_DOWN, NB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
            (void)hipGetLastError();
            return moe_fail(MOE_E_HIP, "moe_ffn_slots: cannot allow %d bytes of LDS for the prefill kernels", lds);
        }
        lds_set = true;
    }
    const int tile_groups = (max_tiles + PF_XCD - 1) / PF_XCD;
    PfArgs gu{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[0], lay.w[1],
              reinterpret_cast<const unsigned char*>(x), pair_list, w, tiles, n_tiles, hbuf, H, I, k, I / (NB * 16)};
    hipLaunchKernelGGL((k_pf_gemm<PF_GU, NB>), dim3((unsigned)(PF_XCD * tile_groups * gu.ntiles_n)),
                       dim3(PF_THREADS), lds, st, gu);
    int rc;
    if ((rc = moe_check_launch("moe_ffn_slots/prefill_gate_up"))) return rc;
    PfArgs dn{reinterpret_cast<const unsigned char*>(slot_store), slab_bytes, lay.w[2], 0,
              reinterpret_cast<const unsigned char*>(hbuf), pair_list, w, tiles, n_tiles, part, I, H, k,
              H / (NB * 32)};
    hipLaunchKernelGGL((k_pf_gemm<PF_DOWN, NB>), dim3((unsigned)(PF_XCD * tile_groups * dn.ntiles_n)),
                       dim3(PF_THREADS), lds, st, dn);
    return moe_check_launch("moe_ffn_slots/prefill_down");
}

}  // namespace

bool moe_pf_supported(int w_type, int H, int I) {
    // column tiles of 64 h columns / 128 output rows; contraction in pairs of 64-wide steps
    return w_type == MOE_W_BF16 && H % 128 == 0 && I % 128 == 0;
}

int moe_pf_tile_rows(int T, int k) { return T * k < PF_BIG_P ? DEC_MT : PF_MT; }

bool moe_pf_big(int T, int k, int S, int H, int I) {
    // hundreds of picks per slot on average, and whole 256-row / 128-column tiles
    const int P = T * k;
    return P >= PF_BIG_P && P / (S > 0 ? S : 1) >= PB_BIG_ROWS && H % PB_NT == 0 && I % 128 == 0;
}

int moe_pf_tile_rows(int T, int k, int S, int H, int I) {
    return moe_pf_big(T, k, S, H, I) ? PB_MT : moe_pf_tile_rows(T, k);
}

int moe_pf_max_tiles(int T, int k, int S) {
    const int P = T * k;
    return (S < P ? S : P) + P / moe_pf_tile_rows(T, k) + 1;  // bounds the sum over slots of ceil(n_s / rows)
}

size_t moe_pf_tiles_bytes(int T, int k, int S) { return (size_t)moe_pf_max_tiles(T, k, S) * sizeof(PfTile) + 16; }

int moe_pf_run(const void* x, const float* w, int T, int k, const void* slot_store, size_t slab_bytes, int S, int H,
               int I, const moe_slab_layout_t& lay, const int32_t* pair_list, void* tiles_ws, void* hbuf, float* part,
               hipStream_t st) {
    const int P = T * k;
    const int max_tiles = moe_pf_max_tiles(T, k, S);
    const PfTile* tiles = reinterpret_cast<const PfTile*>(tiles_ws);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(reinterpret_cast<unsigned char*>(tiles_ws) +
                                                              (size_t)max_tiles * sizeof(PfTile));

    // decode-sized batches (a few picks per slot): 32-row token tiles; large groups: 256-row tiles
    if (P < PF_BIG_P)
        return dec_launch<DEC_NW>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles, max_tiles,
                                  hbuf, part, st);
    if (moe_pf_big(T, k, S, H, I))
        return pb_launch(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles, max_tiles, hbuf,
                         part, st);
    return pf_launch<4>(x, w, k, slot_store, slab_bytes, H, I, lay, pair_list, tiles, n_tiles, max_tiles, hbuf, part,
                        st);
}

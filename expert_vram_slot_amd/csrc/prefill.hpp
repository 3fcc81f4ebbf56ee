// Prefill-sized grouped GEMM path of moe_ffn_slots (bf16 weights, MFMA).
#pragma once

#include "common.hpp"

// A token tile of the grouped GEMM: up to moe_pf_tile_rows() consecutive
// picks of one slot in the slot-sorted pick list.  Written by the
// pick-sorting kernels.
struct moe_pf_tile {
    int p0;    // first position in the slot-sorted pick list
    int rows;  // picks of the tile (1 .. tile rows)
    int slot;
    int pad;
};

// True when the MFMA path handles this weight format and shape.
bool moe_pf_supported(int w_type, int H, int I);
// Workspace bytes of the tile list for T*k picks over S slots (the list,
// then its length as one int32).
size_t moe_pf_tiles_bytes(int T, int k, int S);
// Token rows per tile for a batch of T*k picks: 32 for decode-sized batches
// (a few picks per slot), 128 for prefill-sized ones.
int moe_pf_tile_rows(int T, int k);
int moe_pf_tile_rows(int T, int k, int S, int H, int I);
bool moe_pf_big(int T, int k, int S, int H, int I);
// Token rows per tile for a weight format: int8 weights always take 32-row
// (decode-shaped) tiles; bf16 as moe_pf_tile_rows(T, k, S, H, I).
int moe_pf_tile_rows_for(int w_type, int T, int k, int S, int H, int I);
// Largest number of tiles T*k picks over S slots can need.
int moe_pf_max_tiles(int T, int k, int S);
// True when a batch of T*k picks can be sorted by the gate/up workgroups
// themselves (decode-shaped tiles, at most 1024 picks).
bool moe_pf_fused_sort(int T, int k);
// True when moe_pf_run writes the partials as bf16 (the prefill-shaped
// kernels: bf16 weights, 4096 picks and more); otherwise they are fp32.
bool moe_pf_part_bf16(int w_type, int T, int k);
// Gate/up and down grouped GEMMs over the slot-sorted picks; h goes to hbuf
// in sorted order, w * (W_d h) to part[pick][H] (bf16 or fp32, as
// moe_pf_part_bf16 says).  Enqueued on `st`.  With
// sort_slots == NULL, pair_list and the tile list in tiles_ws were written by
// the sorting kernels; otherwise (moe_pf_fused_sort(T, k) must hold) the
// gate/up kernel sorts the picks by sort_slots (slot per pick) and writes
// both for the down kernel.
// int8 weights (w_type MOE_W_W8A8): x is the int8 codes [T][H] with per-token
// scales xscale[T], h goes to hbuf in fp32 (sorted order) and each gate/up
// column tile's max |h| per pick to hmax[I / 64][P] (sorted order; written in
// full, nothing to clear), decode-shaped tiles at every batch size (the tile
// rows the sort wrote must be 32; no fused sort).
int moe_pf_run(const void* x, const float* w, int T, int k, const void* slot_store, size_t slab_bytes, int S, int H,
               int I, const moe_slab_layout_t& lay, const int32_t* pair_list, void* tiles_ws, void* hbuf,
               float* part, hipStream_t st, const int32_t* sort_slots = nullptr, int w_type = MOE_W_BF16,
               const float* xscale = nullptr, float* hmax = nullptr);

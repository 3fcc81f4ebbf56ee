// Prefill-sized grouped GEMM path of moe_ffn_slots (bf16 weights, MFMA).
#pragma once

#include "common.hpp"

// True when the MFMA path handles this weight format and shape.
bool moe_pf_supported(int w_type, int H, int I);
// Workspace bytes of the tile list for T*k picks over S slots.
size_t moe_pf_tiles_bytes(int T, int k, int S);
// Gate/up and down grouped GEMMs over the slot-sorted picks (slot_off,
// pair_list, active, n_active from the sorting kernel); h goes to hbuf in
// sorted order, w * (W_d h) to part[pick][H].  Enqueued on `st`.
int moe_pf_run(const void* x, const float* w, int T, int k, const void* slot_store, size_t slab_bytes, int S, int H,
               int I, const moe_slab_layout_t& lay, const int32_t* slot_off, const int32_t* pair_list,
               const int32_t* active, const int32_t* n_active, void* tiles_ws, void* hbuf, float* part,
               hipStream_t st);

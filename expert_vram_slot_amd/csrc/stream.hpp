// Streamed miss pass of the native step driver (large batches): the picks of
// non-resident experts are served on the GPU from a ring of staging slots
// that their slabs are gathered into, chunk by chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_slot.h"

int moe_fail(int code, const char* fmt, ...);
int moe_ok();

// pos[p] = index of pick p's expert in host_miss[0 .. *n_host) (ascending
// expert ids) when the pick is not resident (slot_ids[p] < 0), else -1.
int moe_stream_pos(const int32_t* ids, const int32_t* slot_ids, int P, const int32_t* host_miss,
                   const int32_t* n_host, int32_t* pos, hipStream_t st);

// Chunk c of the streamed misses: host_miss[c0 .. c0 + R) go to staging slots
// base .. base + R - 1.  Writes the chunk's gather list (expert, staging
// slot) and its length (device), and the staging slot of every pick of the
// chunk's experts (cslots[p], -1 for every other pick).
int moe_stream_chunk(const int32_t* pos, int P, const int32_t* host_miss, const int32_t* n_host, int c0, int R,
                     int base, int32_t* cmiss, int32_t* n_cmiss, int32_t* cslots, hipStream_t st);

/*
 * moe_slot.h -- C ABI of the MI355X (gfx950) expert-slot MoE layer.
 *
 * One Mixture-of-Experts layer whose experts live in a fixed number of VRAM
 * "slots" in front of a pinned host copy of every expert:
 *
 *   moe_route            router logits, optional graded selection bias, top-k,
 *                        softmax of the raw logits over the picked k
 *   cache_manage         victims among slots this step does not need + miss list,
 *                        fused with the expert-id -> slot remap
 *   cache_gather         missing experts copied from pinned host memory to slots
 *   moe_ffn_slots        grouped SwiGLU FFN over resident slots; picks whose slot
 *                        is -1 contribute exactly zero
 *   moe_ffn_host_misses  the same FFN on CPU threads for the picks that are not
 *                        resident; summed in with moe_combine
 *
 * Sources (web pages, by title and section):
 *   [BEL] the Betelgeuse engine post: an in-stream kernel resolves expert hits
 *         on the device and rings a mapped host doorbell only on a miss.
 *   [RTX] sozai.app transcript "rtx-3060-run-35b-llamacpp" -- "What the video
 *         covers", "Full Transcript": a fixed slot set chosen at load, missing
 *         experts return zeros on the GPU, a CPU pass over the RAM experts, one
 *         add to join them.
 *   [VEC] "Porting vllm-expert-cache to NVIDIA GPUs" -- "What this package does"
 *         (expert_cache_manage, expert_cache_gather, remap to slot space;
 *         expert_cache_fused, named in "The port"),
 *         "The port" (16-byte copy unit, build-time export check, binding by
 *         exported name), "Prove it is correct before measuring" (determinism:
 *         no atomics, no order-dependent reduction; the device reads pinned host
 *         memory; per-expert slabs in 16-byte multiples), "Measuring, without
 *         fooling yourself" (a step is served from slots alone only when it fits),
 *         "What we know, and what we are guessing" (refuse loudly, with a reason;
 *         read source tensors fresh on every call; weights and scales are both
 *         slot-indexed).
 *   [PGO] "Nudge, don't cut" -- "The method in five lines": bias[l][e] =
 *         max(cap, ln(b[l][e] / b_edge[l])), top-k by logit + bias, weights from
 *         the router's own softmax over the picked k; static table; opt-in.
 *         "Experts that don't fit": the hard mask and the flat soft bias;
 *         "Qwen on Strata: the bias as a quality dial": damped weights;
 *         "Then Maya's own knob beat ours": live-cache affinity (a small lambda
 *         on every expert in VRAM now, decode only).
 *
 * Conventions for every entry point
 *   - Return 0 on success or a negative MOE_E_* code; moe_last_error() then
 *     holds a one-line reason (thread-local).  Nothing aborts or exits.
 *   - "device" pointers are HIP device memory (or device-visible pinned host
 *     memory where stated); "host" pointers are CPU memory.  The caller owns
 *     every buffer.  The device calls allocate nothing per call and keep no
 *     pointer to caller memory between calls (the host pass keeps host
 *     scratch of its own, below).
 *   - Device calls enqueue on the given stream and never synchronise with the
 *     host.  Counts produced on the device (n_miss, n_host) stay there.
 *   - Identical inputs give bit-identical outputs (fixed reduction orders, no
 *     floating-point atomics).
 *   - Weights are row-major [out][in]: gate Wg[I][H], up Wu[I][H], down
 *     Wd[H][I]; router gate G[E][H].
 */
#ifndef MOE_SLOT_H
#define MOE_SLOT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* status codes */
#define MOE_OK 0
#define MOE_E_ARG (-1)    /* null pointer, negative or out-of-range size */
#define MOE_E_ALIGN (-2)  /* pointer or slab not 16-byte aligned / a 16-byte multiple */
#define MOE_E_DTYPE (-3)  /* unsupported activation / weight format pair */
#define MOE_E_SHAPE (-4)  /* inconsistent or unsupported shape (k > E, S > E, limits) */
#define MOE_E_HIP (-5)    /* a HIP runtime call or kernel launch failed */
#define MOE_E_NOMEM (-6)  /* a pinned or host allocation failed */

/* activation formats (x and the router gate G) */
#define MOE_X_F32 0
#define MOE_X_BF16 1

/* expert weight formats (one slab per expert, see moe_slab_layout) */
#define MOE_W_F32 0    /* fp32 weights, fp32 activations, h kept in fp32 */
#define MOE_W_BF16 1   /* bf16 weights and activations; h rounded to bf16 (RNE) */
#define MOE_W_W8A8 2   /* int8 weights + fp32 per-output-row scales; x and h
                          quantised per token / per pick to int8 with scale
                          absmax/127 (1 if all zero), code = clamp(rint(v/scale),
                          -127, 127), both in fp32; int32 dots; dequant
                          ((float)acc * s_act) * s_row */
#define MOE_W_Q4B32 3  /* 4-bit blocks of 32 inputs, fp16 scale per block:
                          w = scale * (nibble - 8); x bf16; h rounded to bf16 */

/* cache policies */
#define MOE_STATIC 0   /* resident set fixed at load, never evicted */
#define MOE_LRU 1
#define MOE_LFU 2

/* limits */
#define MOE_MAX_E 4096     /* experts per layer */
#define MOE_MAX_S 1024     /* slots per layer */
#define MOE_MAX_K 32       /* top-k */

/* Cache state of one layer, all device arrays owned by the caller and
 * mutated only by cache_manage / cache_init, in stream order.
 *   e2s[E]   slot of expert e, -1 if not resident
 *   s2e[S]   expert in slot s, -1 if empty
 *   last[S]  step of the slot's last use        (LRU / LFU priority)
 *   freq[S]  uses since the expert entered      (LFU priority)
 *   step[1]  step counter, +1 per cache_manage call */
typedef struct {
    int32_t* e2s;
    int32_t* s2e;
    uint32_t* last;
    uint32_t* freq;
    uint32_t* step;
    int32_t E;
    int32_t S;
} moe_cache_state;

/* Byte offsets inside one expert's slab.  w[p] / s[p] are the weight plane
 * and scale plane of projection p (0 gate, 1 up, 2 down); s[p] = -1 where the
 * format has no scales.
 *   F32 / BF16: Wg | Wu | Wd
 *   W8A8:       Wg | Wu | Wd (int8) | sg[I] | su[I] | sd[H] (fp32)
 *   Q4B32:      per projection, a nibble plane [out][in/2] then an fp16 scale
 *               plane [out][in/32]; order gate, up, down.  Block b of a row
 *               covers inputs 32b..32b+31; byte j of the block holds input
 *               32b+j in its low nibble and 32b+j+16 in its high nibble. */
typedef struct {
    int64_t w[3];
    int64_t s[3];
    int64_t total;
} moe_slab_layout_t;

int moe_abi_version(void);
const char* moe_last_error(void);

/* Slab layout of one expert.  Requires H, I multiples of 16 (32 for Q4B32)
 * so that every plane starts on a 16-byte boundary ([VEC] "Prove it is
 * correct before measuring": per-expert slabs stay 16-byte multiples). */
int moe_slab_layout(int w_type, int H, int I, moe_slab_layout_t* out);

/* Graded selection bias of one layer, [PGO] "The method in five lines".
 *   b      device double[E]: brightness (share of router mass) per expert
 *   n_hot  size of the hot set = the n_hot brightest experts (ties: lower id)
 *   cap    floor of the penalty (e.g. -1)
 *   bias   device float[E] out: 0 for hot experts, else
 *          max(cap, ln(b[e] / b_edge)) with b_edge the weakest hot expert's
 *          brightness, computed in double (b = 0 gives cap).
 * Errors: ARG (null, E < 1, n_hot < 1), SHAPE (E > MOE_MAX_E). */
int moe_bias_table(const double* b, int E, int n_hot, float cap, float* bias, hipStream_t stream);

/* Flat selection bias, or the hard mask, of one layer, [PGO] "Experts that
 * don't fit".  The hot set is the one moe_bias_table uses.
 *   b      device double[E]: brightness per expert
 *   n_hot  the n_hot brightest experts (ties: lower id) get 0
 *   value  every other expert gets this number; <= 0, not NaN.  -INFINITY is
 *          the hard mask: a cold expert never outranks a hot one, so with at
 *          least k hot experts no cold expert is picked.
 *   bias   device float[E] out
 * Errors: ARG (null, E < 1, n_hot < 1, value > 0 or NaN), SHAPE (E > MOE_MAX_E). */
int moe_bias_flat(const double* b, int E, int n_hot, float value, float* bias, hipStream_t stream);

/* Live-cache affinity, [PGO] "Then Maya's own knob beat ours": lambda added to
 * the selection score of every expert that is in VRAM now.
 *   e2s     device int32[E]: a cache state's expert -> slot map, read when the
 *           kernel runs (so in stream order after the last cache_manage)
 *   base    device float[E] or NULL: a static table to add to (NULL reads 0)
 *   lambda  finite
 *   bias    device float[E] out: fl32(base[e] + lambda) where e2s[e] >= 0,
 *           else base[e]; pass it to moe_route as the bias.  The pages use it
 *           at decode only; which calls get it is the caller's choice.
 * Errors: ARG (null, E < 1, lambda not finite), SHAPE (E > MOE_MAX_E). */
int moe_bias_affinity(const int32_t* e2s, const float* base, int E, float lambda, float* bias, hipStream_t stream);

/* Router, [PGO] "The method in five lines".
 *   x       device [T][H] in x_dtype
 *   G       device [E][H] in x_dtype (one row per expert)
 *   bias    device float[E] or NULL.  NULL gives exactly the plain top-k of
 *           the logits (the bias is opt-in).
 *   ids_in  device int32[T][k] or NULL.  If given, the picks are taken as is
 *           (externally sampled routing) and only w (and logits) are produced.
 *   ids     device int32[T][k] out: picks by score s = fl32(z + bias), highest
 *           first, ties to the lower expert id (ignored if ids_in != NULL)
 *   w       device float[T][k] out: softmax of the raw logits z over the k
 *           picks (selection-only bias), computed in double
 *   logits  device float[T][E] out, or NULL: z = x G, accumulated in double
 *           and rounded once to fp32
 * Errors: ARG, DTYPE, SHAPE (k > E, k > MOE_MAX_K, E > MOE_MAX_E), HIP. */
int moe_route(const void* x, int x_dtype, const void* G, const float* bias, const int32_t* ids_in, int T, int H,
              int E, int k, int32_t* ids, float* w, float* logits, hipStream_t stream);

/* moe_route with options; flags = 0 is moe_route exactly.
 *   MOE_ROUTE_DAMPED  w is the softmax over the k picks of the biased scores
 *                     s = fl32(z + bias) ("damped weights", [PGO] "Qwen on
 *                     Strata: the bias as a quality dial") instead of the raw
 *                     logits; with bias NULL the two are the same.
 * Errors: those of moe_route; ARG for an unknown flag. */
#define MOE_ROUTE_DAMPED 1
int moe_route_ex(const void* x, int x_dtype, const void* G, const float* bias, const int32_t* ids_in, int T, int H,
                 int E, int k, int flags, int32_t* ids, float* w, float* logits, hipStream_t stream);

/* Initialise a cache state.  resident: device int32[S] (slot s holds expert
 * resident[s]) or NULL for an empty cache.  Clears last/freq and step.
 * Errors: ARG, SHAPE (S > E, S > MOE_MAX_S, E > MOE_MAX_E). */
int cache_init(const moe_cache_state* st, const int32_t* resident, hipStream_t stream);

/* Static resident set from a profile batch ([RTX] transcript: the set is
 * chosen once, before the run, from what the router picks): the S most-picked
 * experts among ids[n_ids], ties to the lower id, most-picked first.
 *   ids device int32[n_ids]; resident device int32[S] out. */
int cache_pick_static(const int32_t* ids, int n_ids, int E, int S, int32_t* resident, hipStream_t stream);

/* One cache step, [VEC] "What this package does" (expert_cache_manage plus
 * the remap to slot space).  One workgroup, deterministic, no atomics.
 *   st        cache state (mutated)
 *   policy    MOE_STATIC / MOE_LRU / MOE_LFU
 *   ids       device int32[n_ids] routing ids of this step (T*k)
 *   slot_ids  device int32[n_ids] out: slot of ids[i] after the step, -1 if
 *             the expert is not resident (its pick is left to the host pass)
 *   miss      device int32[2*S] out: (expert, slot) pairs to gather, experts
 *             in ascending id; the i-th miss takes the i-th victim
 *   n_miss    device int32[1] out
 *   host_miss device int32[E] out: needed experts left non-resident
 *             (ascending id): all misses under STATIC, the overflow beyond
 *             the victims otherwise
 *   n_host    device int32[1] out
 *   stats     device int32[4] out or NULL: routing ids resident at entry,
 *             distinct experts needed, gathered, host misses
 * Victims are the slots that hold no expert needed this step: empty slots
 * first (lower slot first), then LRU by last use / LFU by use count then last
 * use, ties to the lower slot.  A hit refreshes last (LFU: count + 1 per
 * step); an inserted expert starts at last = step, freq = 1.  STATIC never
 * changes the maps.  Overflow (more misses than victims) is not an error.
 * Errors: ARG, SHAPE (n_ids > 2^24, E or S beyond the limits), HIP. */
int cache_manage(const moe_cache_state* st, int policy, const int32_t* ids, int n_ids, int32_t* slot_ids,
                 int32_t* miss, int32_t* n_miss, int32_t* host_miss, int32_t* n_host, int32_t* stats,
                 hipStream_t stream);

/* Doorbell of a fused cache step in pinned host memory ([BEL]: the in-stream
 * resolve rings a mapped host doorbell, so the host learns of misses without
 * a stream synchronisation).  seq is written last, with system-scope release
 * ordering: a host thread that reads seq == the call's seq (acquire) may read
 * the other fields and the picks mirrored beside it.  n_host == 0 means no
 * pick of the step needs the host pass.  err is never written by the
 * managing workgroup: a copying workgroup that stopped waiting for the cache
 * step sets it to 1 (system scope) and copies nothing, so the caller clears
 * it before the call and reads it once the call's kernel has finished; a
 * nonzero err with n_miss > 0 means the gather is incomplete. */
typedef struct {
    int32_t seq;
    int32_t n_miss;
    int32_t n_host;
    int32_t stats[4];
    int32_t err;
} moe_doorbell;

/* cache_manage and cache_gather in one launch ([VEC] "The port":
 * expert_cache_fused), with an optional doorbell ([BEL] in-stream doorbell).
 * Arguments as cache_manage and cache_gather (host_store pinned; STATIC
 * caches copy nothing), plus:
 *   w           device float[n_ids] or NULL: routing weights to mirror
 *   sync        device int32[2], zeroed once by the caller, owned by this
 *               call sequence (not shared by calls that may overlap): the
 *               in-kernel hand-off from the managing workgroup to the copying
 *               ones; sync[1] is set (never cleared) by a copying workgroup
 *               that gave up waiting: the gather of that call is then
 *               incomplete (with co-resident workgroups this does not happen
 *               within the default wait); the caller clears sync[1] to
 *               re-arm the report
 *   seq         a number new for every call on this sync word and doorbell
 *   bell        pinned host moe_doorbell or NULL
 *   bell_ids, bell_slots, bell_w
 *               pinned host int32/int32/float[n_ids] or NULL: ids, slot_ids
 *               and w mirrored to the host before the doorbell rings
 * One workgroup runs the cache step, mirrors the picks, rings the doorbell
 * and releases the others, which wait for it (bounded) and then copy the
 * missing slabs together with it.  Results equal cache_manage followed by
 * cache_gather.
 * Errors: those of cache_manage and cache_gather; ARG (sync NULL).  A
 * copying workgroup that gives up is reported in sync[1] and bell->err (the
 * call itself has already returned by then). */
int cache_manage_gather(const moe_cache_state* st, int policy, const int32_t* ids, int n_ids, const float* w,
                        int32_t* slot_ids, int32_t* miss, int32_t* n_miss, int32_t* host_miss, int32_t* n_host,
                        int32_t* stats, const void* host_store, void* slot_store, size_t slab_bytes, int32_t* sync,
                        int32_t seq, moe_doorbell* bell, int32_t* bell_ids, int32_t* bell_slots, float* bell_w,
                        hipStream_t stream);

/* How many times a copying workgroup of cache_manage_gather polls the
 * hand-off word (with a short sleep between polls) before it gives up; the
 * default is 2^22 (a fraction of a second).  polls >= 0 sets the limit for
 * later calls in this process (0: every copying workgroup gives up at once,
 * which exercises the report of an incomplete gather without a fault or a
 * hang); polls < 0 only queries.  Returns the limit in force before the
 * call.  Not for concurrent use with calls being enqueued. */
int64_t moe_fused_spin_limit(int64_t polls);

/* Periodic repick of the resident set, [RTX] "Full Transcript" (every ~500
 * tokens have another look, swap out whatever has gone cold, then leave the
 * set alone; a static set between repicks).
 *   want    device int32[S]: the new set (e.g. cache_pick_static over the
 *           last window's picks); a repeated or out-of-range entry is skipped
 *   miss    device int32[2*S] out: (expert, slot) loads for cache_gather
 *   n_miss  device int32 out: number of loads
 * Members of the new set already resident keep their slots; the others are
 * loaded, in ascending expert id, into the slots whose expert is not in the
 * new set (empty slots included), in ascending slot order; a slot no load
 * needs keeps its expert.  A loaded slot restarts with last = step, freq = 0;
 * step does not advance.  Follow with cache_gather(miss, n_miss, S, ...).
 * Errors: ARG, SHAPE (as cache_manage). */
int cache_repick(const moe_cache_state* st, const int32_t* want, int32_t* miss, int32_t* n_miss, hipStream_t stream);

/* Copy each missing expert's slab from pinned host memory into its slot,
 * [VEC] "What this package does" / "The port": the device itself reads the
 * host memory, in 16-byte units.  Launch it on a side stream and order the
 * FFN after it with an event.
 *   miss        device int32[2*max_miss] (from cache_manage)
 *   n_miss      device int32[1] (read on the device; no host sync)
 *   host_store  pinned host memory [E][slab_bytes] (hipHostMalloc /
 *               moe_host_alloc / torch pinned tensor); its device address is
 *               looked up on every call
 *   slot_store  device [S][slab_bytes]
 * Errors: ARG (host_store not pinned), ALIGN (pointers or slab_bytes not
 * 16-byte multiples), HIP. */
int cache_gather(const int32_t* miss, const int32_t* n_miss, int max_miss, const void* host_store, void* slot_store,
                 size_t slab_bytes, hipStream_t stream);

/* Workspace bytes moe_ffn_slots needs for these sizes (device memory the
 * caller allocates once and passes in). */
size_t moe_ffn_workspace_bytes(int T, int k, int S, int w_type, int H, int I);

/* Grouped SwiGLU FFN over the resident slots ([RTX] transcript: the expert
 * step returns zeros for an expert that is not on the GPU).
 *   x         device [T][H] in x_dtype (MOE_X_F32 for MOE_W_F32, else bf16)
 *   slot_ids  device int32[T][k]; -1 = not resident: that pick adds exactly 0
 *   w         device float[T][k] routing weights
 *   slot_store device [S][slab_bytes] (16-byte aligned; slab_bytes >= layout)
 *   y         device float[T][H] out (overwritten):
 *             y[t] = sum over j with slot_ids[t][j] >= 0 of w[t][j] * FFN_slot(x[t]),
 *             summed in j order in fp32; +0.0 where token t has no resident
 *             pick.  With bf16 weights and T*k >= 4096 each term is rounded
 *             once to bf16 before the sum (prefill-sized batches)
 *   ws        device workspace of >= moe_ffn_workspace_bytes(...) bytes
 * Errors: ARG, ALIGN, DTYPE, SHAPE, HIP. */
int moe_ffn_slots(const void* x, int x_dtype, const int32_t* slot_ids, const float* w, int T, int k,
                  const void* slot_store, size_t slab_bytes, int S, int w_type, int H, int I, float* y, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* moe_ffn_slots without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results (bit for bit) and
 * errors as moe_ffn_slots.  The workspace is a static device array of
 * moe_ffn_noalloc_scratch_bytes() = 32 MiB in the library's code object: each
 * GPU the library runs on holds its own copy until the process ends, and the
 * call allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine).  Sizes whose workspace (moe_ffn_workspace_bytes) exceeds it are
 * refused with SHAPE before anything is enqueued: decode batches fit (the
 * 128-expert, top-8, 2048 x 768 bf16 layer up to about 400 tokens), prefill
 * batches of thousands of tokens do not.  The scratch keeps the last call's
 * contents; no part of it needs to start at zero.  Calls that may overlap on
 * one GPU (different streams, or different host threads) share the array
 * and race: serialise them.  HIP when the array's device address cannot be
 * found on the current device. */
int moe_ffn_slots_noalloc(const void* x, int x_dtype, const int32_t* slot_ids, const float* w, int T, int k,
                          const void* slot_store, size_t slab_bytes, int S, int w_type, int H, int I, float* y,
                          hipStream_t stream);
/* Bytes of the static workspace of moe_ffn_slots_noalloc (for callers that
 * cannot allocate device memory). */
size_t moe_ffn_noalloc_scratch_bytes(void);

/* Host pass over the picks that are not resident, [RTX] "What the video
 * covers" / transcript (a CPU pass over the experts still in RAM).  Runs
 * synchronously on the calling thread plus n_threads - 1 workers; safe to
 * run while the GPU calls are in flight.
 *   x_h, ids_h, slot_ids_h, w_h  host copies of x [T][H], ids [T][k],
 *                                slot_ids [T][k], w [T][k]
 *   host_store                   host [E][slab_bytes] (pinned or not)
 *   y_h                          host float[T][H] out (overwritten):
 *                                sum over j with slot_ids[t][j] < 0 of
 *                                w[t][j] * FFN_ids[t][j](x[t]), in j order
 * Same per-format arithmetic as moe_ffn_slots.  Intermediate rows (about
 * T*k*(4H + 6I) bytes) live in host scratch kept per calling thread between
 * calls, so repeated steps neither zero-fill nor fault them in again; a
 * buffer above 64 MiB is released when its call returns.  Errors: ARG,
 * DTYPE, SHAPE, NOMEM (the scratch cannot be allocated). */
int moe_ffn_host_misses(const void* x_h, int x_dtype, const int32_t* ids_h, const int32_t* slot_ids_h,
                        const float* w_h, int T, int k, const void* host_store, size_t slab_bytes, int E, int w_type,
                        int H, int I, float* y_h, int n_threads);

/* y[i] = fl32(y[i] + y_add[i]) for T*H floats on the device: the single add
 * that joins the two passes ([RTX] transcript). */
int moe_combine(float* y, const float* y_add, int T, int H, hipStream_t stream);

/* Residual join of stacked layers ([PGO] "Experts that don't fit": the
 * routed layers follow one another in a deep model; each adds its output to
 * the activations it read):
 *   x      device [T][H] in x_dtype (MOE_X_BF16 or MOE_X_F32)
 *   y      device float[T][H], the layer's output
 *   x_out  device [T][H] in x_dtype out; may alias x
 * bf16: x_out = RNE_bf16(fl32(x + y)); fp32: x_out = fl32(x + y).
 * Errors: ARG, DTYPE, HIP. */
int moe_residual(const void* x, int x_dtype, const float* y, void* x_out, int T, int H, hipStream_t stream);

/* Pinned, device-mapped host memory for the host expert store. */
void* moe_host_alloc(size_t bytes);
int moe_host_free(void* p);

/* ------------------------------------------------------------------------
 * Native step driver.  The entry points above issued in the order of one
 * layer step ([RTX] "Full Transcript": the GPU work of a layer runs as one
 * unbroken sequence while the CPU runs the experts that stay in RAM; one add
 * joins them.  [VEC] "What this package does": manage, gather and remap
 * before the expert FFN), without an interpreter between the calls.
 *
 * A layer as the driver sees it (every pointer owned by the caller):
 *   G           device [E][H] router gate (activation format)
 *   bias        device float[E] selection bias or NULL
 *   state       the layer's cache state (device arrays)
 *   policy      MOE_STATIC / MOE_LRU / MOE_LFU
 *   slot_store  device [S][slab_bytes]
 *   host_store  pinned, device-mapped host [E][slab_bytes]
 */
typedef struct {
    const void* G;
    const float* bias;
    moe_cache_state state;
    int policy;
    void* slot_store;
    const void* host_store;
    size_t slab_bytes;
} moe_layer_desc;

/* Buffers, events and pinned staging of one step shape (T <= T_max tokens
 * over E experts, top-k, S slots, one weight format).  Created once: this is
 * where the driver allocates (device memory, pinned host memory, events);
 * the step calls allocate nothing.  NULL on failure (reason in
 * moe_last_error). */
typedef struct moe_step moe_step;
moe_step* moe_step_create(int T_max, int E, int k, int H, int I, int S, int w_type);
void moe_step_destroy(moe_step* h);
/* device float[T_max][H]: y of the last moe_layer_step called with
 * y_out = NULL (valid in stream order). */
const float* moe_step_output(const moe_step* h);
/* Cache counters (cache_manage's stats: routing ids resident at entry,
 * distinct experts needed, gathered, host misses) summed over the steps run
 * with the host pass; out int64[4]; reset != 0 clears the sums. */
int moe_step_stats(moe_step* h, int64_t* out, int reset);

/* One layer step for T tokens of x (device [T][H], activation format):
 * moe_route (ids_in: given device picks [T][k] or NULL) -> the cache step ->
 * moe_ffn_slots on s0.  With host_pass != 0 the cache step is
 * cache_manage_gather (one launch: cache step, gather of the misses, and the
 * picks mirrored to pinned memory behind a doorbell); x goes to pinned
 * memory on s_copy while the router runs; this thread waits for the
 * doorbell and, only when the step has host misses, serves them in one of
 * two ways ([RTX] "Full Transcript": the concurrent CPU lane pays off on
 * small batches; on a big prompt batch it is switched off):
 *  - the CPU lane: moe_ffn_host_misses on n_threads threads while the GPU
 *    runs the FFN, the result added on s0 (moe_combine);
 *  - streamed (large batches, when the host picks reach the step's
 *    threshold per non-resident expert, see moe_step_set_stream_threshold):
 *    the non-resident experts' slabs are gathered, 8 at a time, into a ring
 *    of 16 staging slots on s_side, each chunk's gather overlapping the FFN
 *    of the previous chunk on s0, and each chunk's FFN result is added to y.
 *    Only steps created with T_max >= 128 have the ring.
 * When the step gathered slabs into its slots, the call waits for the cache
 * step's kernel to finish (normally long done by then) and checks its
 * doorbell for a copying workgroup that gave up.  Without the host pass the
 * cache step is cache_manage, followed by cache_gather for a dynamic cache,
 * all on s0 (the FFN needs the gathered slabs; no host wait at all), and
 * non-resident picks add zero.  y_out: device float[T][H] out, or NULL for
 * the driver's own buffer (moe_step_output); final in s0's order when the
 * call returns.  s0, s_side and s_copy are streams of one device (s0 and
 * s_copy distinct).
 * Errors: those of the entry points it calls; SHAPE when the layer does not
 * match the step; HIP when the doorbell stays silent for 10 s, or when a
 * copying workgroup of the cache step gave up (the gather of this step is
 * incomplete: the layer's slot store no longer matches its cache state,
 * which must be initialised again with cache_init). */
int moe_layer_step(moe_step* h, const moe_layer_desc* layer, const void* x, int T, const int32_t* ids_in,
                   int host_pass, int n_threads, float* y_out, hipStream_t s0, hipStream_t s_side,
                   hipStream_t s_copy);

/* Threshold of the streamed miss pass: a step streams its non-resident
 * experts when its non-resident picks number at least picks_per_expert per
 * non-resident expert (default 32: on the 288-expert bf16 layer with 144
 * resident the CPU lane took 95 ms at 28 picks per expert and 185 ms at 57,
 * the streamed pass 100-104 ms).  0 streams every step that has host misses
 * (given a ring); a negative value never streams. */
int moe_step_set_stream_threshold(moe_step* h, int picks_per_expert);
/* How the last moe_layer_step served its non-resident picks: 0 none (or no
 * host pass), 1 the CPU lane, 2 streamed through the GPU; -1 for NULL. */
int moe_step_last_host_mode(const moe_step* h);

/* n_layers layer steps joined by moe_residual: x_{l+1} = x_l + y_l in the
 * activation format ([PGO] "Experts that don't fit": a deep model of routed
 * layers).  x_out: device [T][H] out, the last layer's residual output (may
 * not alias x). */
int moe_stack_step(moe_step* h, const moe_layer_desc* layers, int n_layers, const void* x, int T, int host_pass,
                   int n_threads, void* x_out, hipStream_t s0, hipStream_t s_side, hipStream_t s_copy);

#ifdef __cplusplus
}
#endif
#endif

/*
 * CPU oracle for one MoE layer over an expert-slot cache -- TEST
 * INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does.
 *
 * Plain, single-threaded, slow C: every function is the textbook definition
 * of one step, in double precision unless a stored format or a quantisation
 * decision fixes the precision.  It shares no code, header or table with the
 * GPU library.
 *
 * Sources (web pages, cited by title and section):
 *   [PGO]  "Nudge, don't cut" (oois.ee/pgo-sgb): "The method in five lines",
 *          "PGO-SGB in two pictures", "Experts that don't fit" (hard mask,
 *          flat soft bias), "Qwen on Strata: the bias as a quality dial"
 *          (damped weights), "Then Maya's own knob beat ours" (live-cache
 *          affinity).
 *   [VEC]  "Porting vllm-expert-cache to NVIDIA GPUs" (davetha/vllm-expert-cache
 *          docs/porting-nvidia.md): "What this package does", "Prove it is
 *          correct before measuring", "Measuring, without fooling yourself".
 *   [RTX]  sozai.app transcript "rtx-3060-run-35b-llamacpp": "What the video
 *          covers", "Full Transcript" (zero-return experts, two passes summed).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_X_F32 = 0, ORC_X_BF16 = 1 };
enum { ORC_W_F32 = 0, ORC_W_BF16 = 1, ORC_W_W8A8 = 2, ORC_W_Q4B32 = 3 };
enum { ORC_STATIC = 0, ORC_LRU = 1, ORC_LFU = 2 };

int64_t oracle_slab_bytes(int w_type, int H, int I);

/* Decode the stored weights of one expert to float (exact for every format).
 * wg, wu: [I][H]; wd: [H][I]. */
int oracle_decode_expert(int w_type, const uint8_t* slab, int H, int I, float* wg, float* wu, float* wd);

/* z[t][e] = sum_h x[t][h] G[e][h], accumulated in double, rounded once. */
int oracle_logits(const void* x, int x_dtype, const void* G, int T, int H, int E, float* z);

/* Graded selection bias of one layer ([PGO] "The method in five lines"). */
int oracle_bias_table(const double* b, int E, int n_hot, float cap, float* bias);

/* top-k of fl32(z + bias) per token, ties to the lower expert id. */
int oracle_topk(const float* z, const float* bias, int T, int E, int k, int32_t* ids);

/* softmax of the raw logits restricted to the picked k (double -> fp32). */
int oracle_route_weights(const float* z, const int32_t* ids, int T, int E, int k, float* w);
int oracle_bias_flat(const double* b, int E, int n_hot, float value, float* bias);
int oracle_bias_affinity(const int32_t* e2s, const float* base, int E, float lambda, float* bias);
int oracle_route_weights_damped(const float* z, const float* bias, const int32_t* ids, int T, int E, int k, float* w);

/* One expert's down-projection output for one token, o = Wd h, before the
 * routing weight (double). */
int oracle_expert(int w_type, const uint8_t* slab, int H, int I, const void* x_row, int x_dtype, double* o);

/* Full layer and its split into resident / non-resident passes. */
int oracle_layer(int w_type, const uint8_t* store, int64_t slab_bytes, int E, int H, int I, const void* x,
                 int x_dtype, const int32_t* ids, const int32_t* slot_ids, const float* w, int T, int k,
                 float* y_full, float* y_gpu, float* y_host);

/* Cache bookkeeping for one step ([VEC] "What this package does"). */
int oracle_manage(int policy, int E, int S, int32_t* e2s, int32_t* s2e, uint32_t* last, uint32_t* freq,
                  uint32_t* step, const int32_t* ids, int n_ids, int32_t* slot_ids, int32_t* miss, int32_t* n_miss,
                  int32_t* host_miss, int32_t* n_host, int32_t* stats);

/* Copy each missing expert's slab into its slot, byte for byte. */
int oracle_gather(const int32_t* miss, int n_miss, const uint8_t* host_store, uint8_t* slot_store,
                  int64_t slab_bytes);

/* Residual join of stacked layers: bf16(x + y) for bf16 streams, x + y for fp32. */
int oracle_residual(const void* x, int x_dtype, const float* y, int T, int H, void* out);

/* Static resident set: the S most-picked experts of a profile batch. */
int oracle_pick_static(const int32_t* ids, int n_ids, int E, int S, int32_t* resident);
int oracle_repick(int E, int S, int32_t* e2s, int32_t* s2e, uint32_t* last, uint32_t* freq,
                  const uint32_t* step, const int32_t* want, int32_t* miss, int32_t* n_miss);

#ifdef __cplusplus
}
#endif
#endif

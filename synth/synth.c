/*
 * Seeded synthetic inputs for the MoE expert-slot layer.
 *
 * This module only manufactures inputs: random tensors, their stored
 * encodings (fp32, bf16, int8 with per-row scales, 4-bit blocks of 32 with an
 * fp16 scale), Dirichlet brightness profiles and Zipf-popular routing ids.
 * It contains none of the layer's own arithmetic (no routing, no cache
 * bookkeeping, no expert FFN).  Both the CPU oracle and the GPU path consume
 * exactly the bytes written here.
 *
 * Random numbers: SplitMix64 used as a counter-based generator.  The i-th
 * 64-bit draw of a stream with key K is mix(K + (i + 1) * GAMMA), where mix is
 * SplitMix64's output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Normals use the Box-Muller
 * transform on pairs of draws.  Gamma variates for the Dirichlet use
 * Marsaglia and Tsang (ACM TOMS 26(3), 2000) with the alpha < 1 boost
 * Gamma(alpha) = Gamma(alpha + 1) * U^(1/alpha).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <immintrin.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform in (0, 1), never 0 or 1 */
static inline double unit(uint64_t u) { return ((double)(u >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Key of a tensor: (base seed, tag, layer, expert) folded through the mixer. */
uint64_t synth_key(uint64_t base, uint64_t tag, uint64_t layer, uint64_t expert) {
    uint64_t k = mix64(base + GAMMA);
    k = mix64(k ^ (tag * 0xD1B54A32D192ED03ULL));
    k = mix64(k ^ (layer * 0xAEF17502108EF2D9ULL));
    k = mix64(k ^ (expert * 0xDB4F0B9175AE2165ULL + 1));
    return k;
}

/* Normal draw number i of stream `key` (Box-Muller on draws 2p and 2p+1). */
static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = unit(draw(key, 2 * p));
    double u2 = unit(draw(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* ---------------------------------------------------------------- threads */

typedef struct {
    void (*fn)(void* ctx, int64_t lo, int64_t hi);
    void* ctx;
    int64_t lo, hi;
} job_t;

static void* job_run(void* p) {
    job_t* j = (job_t*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

/* Split [0, n) into nthreads contiguous ranges.  Results never depend on the
 * thread count because every element is a pure function of its index. */
static void parallel_for_min(int64_t n, int nthreads, int64_t min_n, void (*fn)(void*, int64_t, int64_t),
                             void* ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (n < min_n || nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[64];
    job_t jobs[64];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t lo = t * chunk, hi = lo + chunk;
        if (lo >= n) break;
        if (hi > n) hi = n;
        jobs[t].fn = fn; jobs[t].ctx = ctx; jobs[t].lo = lo; jobs[t].hi = hi;
        if (pthread_create(&th[t], NULL, job_run, &jobs[t]) != 0) {
            job_run(&jobs[t]);
            th[t] = 0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
}

static void parallel_for(int64_t n, int nthreads, void (*fn)(void*, int64_t, int64_t), void* ctx) {
    parallel_for_min(n, nthreads, 4096, fn, ctx);
}

/* ------------------------------------------------------- dense tensors */

typedef struct { uint64_t key; double sigma; void* out; } dense_ctx;

static void fill_f32(void* c, int64_t lo, int64_t hi) {
    dense_ctx* d = (dense_ctx*)c;
    float* o = (float*)d->out;
    for (int64_t i = lo; i < hi; ++i) o[i] = (float)(d->sigma * normal_at(d->key, (uint64_t)i));
}

static void fill_bf16(void* c, int64_t lo, int64_t hi) {
    dense_ctx* d = (dense_ctx*)c;
    uint16_t* o = (uint16_t*)d->out;
    for (int64_t i = lo; i < hi; ++i) o[i] = f32_to_bf16_rne((float)(d->sigma * normal_at(d->key, (uint64_t)i)));
}

/* n draws of N(0, sigma^2), rounded to fp32 (dtype 0) or to bf16 RNE (dtype 1). */
int synth_normal(uint64_t key, int64_t n, double sigma, int dtype, void* out, int nthreads) {
    dense_ctx c = {key, sigma, out};
    if (dtype == 0) parallel_for(n, nthreads, fill_f32, &c);
    else if (dtype == 1) parallel_for(n, nthreads, fill_bf16, &c);
    else return -1;
    return 0;
}

/* --------------------------------------------------- expert slab writer */
/*
 * Slab = one expert's gate W_g[I][H], up W_u[I][H] and down W_d[H][I]
 * (row-major [out][in]) in one contiguous block.
 *   type 0 fp32:  Wg | Wu | Wd                                  (4 B each)
 *   type 1 bf16:  Wg | Wu | Wd                                  (2 B each)
 *   type 2 int8:  Wg | Wu | Wd (int8) | sg[I] | su[I] | sd[H]   (fp32 scales)
 *   type 3 q4b32: per projection a nibble plane [out][in/2] then an fp16
 *                 scale plane [out][in/32]; order gate, up, down.
 *                 Block b of row r covers inputs 32b..32b+31; byte j of the
 *                 block holds input 32b+j in its low nibble and 32b+j+16 in
 *                 its high nibble; value = scale * (nibble - 8).
 * Encoders: bf16 round-to-nearest-even; int8 symmetric per output row with
 * scale absmax/127 and round-half-even, clamped to +-127; q4 scale =
 * fp16(absmax/7), code = clamp(rint(w/scale), -8, 7) + 8 (scale 0 -> code 8).
 */

int64_t synth_slab_bytes(int type, int H, int I) {
    int64_t n = (int64_t)H * I;
    switch (type) {
        case 0: return 3 * n * 4;
        case 1: return 3 * n * 2;
        case 2: return 3 * n + 4 * (2 * (int64_t)I + H);
        case 3: return 3 * (n / 2 + n / 16);
        default: return -1;
    }
}

typedef struct {
    int type, H, I;
    double sigma;
    uint64_t base;
    int layer, e0;
    uint8_t* out;
    int64_t slab;
} slab_ctx;

/* Encode row r of a projection (cols values in tmp) into its stored form. */
static void encode_row(int type, int r, int cols, const float* tmp, uint8_t* w, uint8_t* sc) {
        if (type == 0) {
            memcpy(w + (size_t)r * cols * 4, tmp, (size_t)cols * 4);
        } else if (type == 1) {
            uint16_t* o = (uint16_t*)(w + (size_t)r * cols * 2);
            for (int i = 0; i < cols; ++i) o[i] = f32_to_bf16_rne(tmp[i]);
        } else if (type == 2) {
            float amax = 0.f;
            for (int i = 0; i < cols; ++i) { float a = fabsf(tmp[i]); if (a > amax) amax = a; }
            float s = amax > 0.f ? amax / 127.0f : 1.0f;
            int8_t* o = (int8_t*)(w + (size_t)r * cols);
            for (int i = 0; i < cols; ++i) {
                float q = rintf(tmp[i] / s);
                if (q > 127.f) q = 127.f;
                if (q < -127.f) q = -127.f;
                o[i] = (int8_t)q;
            }
            memcpy(sc + (size_t)r * 4, &s, 4);
        } else {
            uint8_t* o = w + (size_t)r * (cols / 2);
            uint16_t* so = (uint16_t*)(sc + (size_t)r * (cols / 32) * 2);
            for (int b = 0; b < cols / 32; ++b) {
                const float* v = tmp + 32 * b;
                float amax = 0.f;
                for (int i = 0; i < 32; ++i) { float a = fabsf(v[i]); if (a > amax) amax = a; }
                uint16_t dh = _cvtss_sh(amax / 7.0f, _MM_FROUND_TO_NEAREST_INT);
                float d = _cvtsh_ss(dh);
                uint8_t q[32];
                for (int i = 0; i < 32; ++i) {
                    int qi = 8;
                    if (d != 0.f) {
                        float t = rintf(v[i] / d);
                        if (t > 7.f) t = 7.f;
                        if (t < -8.f) t = -8.f;
                        qi = (int)t + 8;
                    }
                    q[i] = (uint8_t)qi;
                }
                for (int j = 0; j < 16; ++j) o[16 * b + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
                so[b] = dh;
            }
        }
}

/* one projection matrix [rows][cols] of expert e drawn from stream `key` */
static void encode_proj(const slab_ctx* c, uint64_t key, int rows, int cols, uint8_t* w, uint8_t* sc, float* tmp) {
    for (int r = 0; r < rows; ++r) {
        for (int i = 0; i < cols; ++i) tmp[i] = (float)(c->sigma * normal_at(key, (uint64_t)r * cols + i));
        encode_row(c->type, r, cols, tmp, w, sc);
    }
}

/* offsets of (gate, up, down) weight planes and scale planes inside a slab */
static void slab_offsets(int type, int H, int I, int64_t off[6]) {
    int64_t n = (int64_t)H * I;
    for (int i = 0; i < 6; ++i) off[i] = 0;
    if (type == 0 || type == 1) {
        int es = type == 0 ? 4 : 2;
        off[0] = 0; off[1] = n * es; off[2] = 2 * n * es;
    } else if (type == 2) {
        off[0] = 0; off[1] = n; off[2] = 2 * n;
        off[3] = 3 * n; off[4] = 3 * n + 4 * (int64_t)I; off[5] = 3 * n + 8 * (int64_t)I;
    } else {
        int64_t pq = n / 2, ps = n / 16;
        off[0] = 0; off[3] = pq;
        off[1] = pq + ps; off[4] = 2 * pq + ps;
        off[2] = 2 * (pq + ps); off[5] = 3 * pq + 2 * ps;
    }
}

/* Encode caller-given float matrices Wg[I][H], Wu[I][H], Wd[H][I] into one
 * slab (used to build hand-made test weights). */
int synth_encode_slab(int type, int H, int I, const float* wg, const float* wu, const float* wd, void* out) {
    if (type < 0 || type > 3) return -1;
    if (type == 3 && (H % 32 || I % 32)) return -3;
    int64_t off[6];
    slab_offsets(type, H, I, off);
    uint8_t* s = (uint8_t*)out;
    const float* src[3] = {wg, wu, wd};
    int rows[3] = {I, I, H}, cols[3] = {H, H, I};
    for (int p = 0; p < 3; ++p)
        for (int r = 0; r < rows[p]; ++r)
            encode_row(type, r, cols[p], src[p] + (size_t)r * cols[p], s + off[p], s + off[3 + p]);
    return 0;
}

enum { TAG_WG = 3, TAG_WU = 4, TAG_WD = 5 };

static void slab_one(const slab_ctx* c, int e, float* tmp) {
    uint8_t* s = c->out + (size_t)(e - c->e0) * c->slab;
    int64_t off[6];
    slab_offsets(c->type, c->H, c->I, off);
    uint64_t kg = synth_key(c->base, TAG_WG, c->layer, e);
    uint64_t ku = synth_key(c->base, TAG_WU, c->layer, e);
    uint64_t kd = synth_key(c->base, TAG_WD, c->layer, e);
    encode_proj(c, kg, c->I, c->H, s + off[0], s + off[3], tmp);
    encode_proj(c, ku, c->I, c->H, s + off[1], s + off[4], tmp);
    encode_proj(c, kd, c->H, c->I, s + off[2], s + off[5], tmp);
}

static void slab_range(void* p, int64_t lo, int64_t hi) {
    slab_ctx* c = (slab_ctx*)p;
    int w = c->H > c->I ? c->H : c->I;
    float* tmp = (float*)malloc((size_t)w * sizeof(float));
    if (!tmp) return;
    for (int64_t e = lo; e < hi; ++e) slab_one(c, (int)(c->e0 + e), tmp);
    free(tmp);
}

/* Write the slabs of experts [e0, e1) of one layer into `out` (consecutive,
 * `slab_bytes` apart).  Weights ~ N(0, sigma^2) before encoding.  Work is
 * split over experts; an expert's bytes depend on (base, layer, e) only. */
int synth_slabs(int type, uint64_t base, int layer, int e0, int e1, int H, int I, double sigma, void* out,
                int64_t slab_bytes, int nthreads) {
    if (type < 0 || type > 3 || H <= 0 || I <= 0 || e1 < e0) return -1;
    if (slab_bytes < synth_slab_bytes(type, H, I)) return -2;
    if (type == 3 && (H % 32 || I % 32)) return -3;
    slab_ctx c = {type, H, I, sigma, base, layer, e0, (uint8_t*)out, slab_bytes};
    parallel_for_min(e1 - e0, nthreads, 1, slab_range, &c);
    return 0;
}

/* ----------------------------------------------- brightness (Dirichlet) */

typedef struct { uint64_t key, i; } seq_t;

static double seq_unit(seq_t* s) { return unit(draw(s->key, s->i++)); }

static double seq_normal(seq_t* s) {
    double u1 = seq_unit(s), u2 = seq_unit(s);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* Gamma(a, 1) for a >= 1 by Marsaglia-Tsang squeeze/acceptance */
static double gamma_ge1(seq_t* s, double a) {
    double d = a - 1.0 / 3.0, c = 1.0 / sqrt(9.0 * d);
    for (;;) {
        double z = seq_normal(s), v = 1.0 + c * z;
        if (v <= 0.0) continue;
        v = v * v * v;
        double u = seq_unit(s);
        if (log(u) < 0.5 * z * z + d - d * v + d * log(v)) return d * v;
    }
}

/* E draws of Dirichlet(alpha, ..., alpha) in double (alpha < 1 uses the
 * U^(1/alpha) boost, done in log space so tiny values do not underflow to a
 * zero sum). */
int synth_dirichlet(uint64_t key, int E, double alpha, double* out) {
    if (E <= 0 || !(alpha > 0)) return -1;
    seq_t s = {key, 0};
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    if (!lg) return -2;
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e) {
        if (alpha < 1.0) {
            double g = gamma_ge1(&s, alpha + 1.0);
            double u = seq_unit(&s);
            lg[e] = log(g) + log(u) / alpha;
        } else {
            lg[e] = log(gamma_ge1(&s, alpha));
        }
        if (lg[e] > mx) mx = lg[e];
    }
    double sum = 0.0;
    for (int e = 0; e < E; ++e) { out[e] = exp(lg[e] - mx); sum += out[e]; }
    for (int e = 0; e < E; ++e) out[e] /= sum;
    free(lg);
    return 0;
}

/* ----------------------------------------------- Zipf-popular routing ids */

/* Routing ids for T tokens, k distinct experts each.  Popularity of rank r
 * (1-based) is proportional to r^-s; ranks map to experts through a
 * Fisher-Yates permutation drawn from `key_perm`.  Each token draws k experts
 * one at a time without replacement, each with probability proportional to
 * the popularity among those not yet drawn (inverse-CDF walk on a uniform
 * from `key_draw`).  ids[t*k + j] is the j-th expert drawn for token t. */
int synth_zipf_ids(uint64_t key_perm, uint64_t key_draw, int T, int E, int k, double s, int32_t* ids) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* used = (unsigned char*)malloc((size_t)E);
    if (!perm || !p || !used) { free(perm); free(p); free(used); return -2; }
    seq_t sp = {key_perm, 0};
    for (int i = 0; i < E; ++i) perm[i] = i;
    for (int i = E - 1; i > 0; --i) {
        int j = (int)(seq_unit(&sp) * (double)(i + 1));
        if (j > i) j = i;
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    /* p[e] = popularity of expert e */
    for (int r = 0; r < E; ++r) p[perm[r]] = pow((double)(r + 1), -s);
    for (int t = 0; t < T; ++t) {
        memset(used, 0, (size_t)E);
        double left = 0.0;
        for (int e = 0; e < E; ++e) left += p[e];
        for (int j = 0; j < k; ++j) {
            double u = unit(draw(key_draw, (uint64_t)t * (uint64_t)k + (uint64_t)j)) * left;
            int pick = -1;
            double acc = 0.0;
            for (int e = 0; e < E; ++e) {
                if (used[e]) continue;
                acc += p[e];
                pick = e;
                if (u < acc) break;
            }
            used[pick] = 1;
            left -= p[pick];
            ids[(size_t)t * k + j] = pick;
        }
    }
    free(perm); free(p); free(used);
    return 0;
}

/*
 * CPU oracle for one MoE layer over an expert-slot cache -- TEST
 * INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
 * baseline load it; the product path never does).
 *
 * Every function is the plain definition of one step, single-threaded, in
 * double precision unless a stored format or a quantisation decision fixes
 * the precision.  Page citations are by title and section; see oracle.h.
 *
 * Parity pins: every function here is pinned by the CPU-only tests to
 * closed forms, brute force, textbook algorithms or library routines; see
 * tests/test_oracle_pins.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ formats */

static float bf16_value(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* IEEE 754 binary16 -> float, from the format's definition. */
static float half_value(uint16_t h) {
    int sign = h >> 15, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(man | 0x400), ex - 25);
    return (float)(sign ? -v : v);
}

/* Round a float to bf16 (nearest, ties to even) and return it as float. */
static float round_bf16(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;
    float r;
    memcpy(&r, &b, 4);
    return r;
}

int64_t oracle_slab_bytes(int w_type, int H, int I) {
    int64_t n = (int64_t)H * I;
    if (w_type == ORC_W_F32) return 12 * n;
    if (w_type == ORC_W_BF16) return 6 * n;
    if (w_type == ORC_W_W8A8) return 3 * n + 4 * (2 * (int64_t)I + H);
    if (w_type == ORC_W_Q4B32) return (3 * n * 18) / 32;
    return -1;
}

/* A read-only view of one expert's slab: projection p (0 gate, 1 up, 2 down)
 * has `rows` outputs and `cols` inputs. */
typedef struct {
    int w_type, H, I;
    const uint8_t* w[3];  /* weight plane of each projection */
    const uint8_t* s[3];  /* scale plane (int8: fp32 [rows], q4: fp16 [rows][cols/32]) */
} expert_view;

static void view_expert(expert_view* v, int w_type, const uint8_t* slab, int H, int I) {
    int64_t n = (int64_t)H * I;
    v->w_type = w_type; v->H = H; v->I = I;
    if (w_type == ORC_W_F32 || w_type == ORC_W_BF16) {
        int es = w_type == ORC_W_F32 ? 4 : 2;
        for (int p = 0; p < 3; ++p) { v->w[p] = slab + p * n * es; v->s[p] = NULL; }
    } else if (w_type == ORC_W_W8A8) {
        for (int p = 0; p < 3; ++p) v->w[p] = slab + p * n;
        v->s[0] = slab + 3 * n;
        v->s[1] = slab + 3 * n + 4 * (int64_t)I;
        v->s[2] = slab + 3 * n + 8 * (int64_t)I;
    } else {
        /* per projection: nibbles [rows][cols/2], then fp16 scales [rows][cols/32] */
        int64_t nib = n / 2, sc = n / 16;
        for (int p = 0; p < 3; ++p) {
            v->w[p] = slab + p * (nib + sc);
            v->s[p] = v->w[p] + nib;
        }
    }
}

static int proj_cols(const expert_view* v, int p) { return p == 2 ? v->I : v->H; }

static float row_scale_i8(const expert_view* v, int p, int r) {
    float s;
    memcpy(&s, v->s[p] + 4 * (int64_t)r, 4);
    return s;
}

/* Exact float value of weight (r, c) of projection p. */
static float weight(const expert_view* v, int p, int r, int c) {
    int cols = proj_cols(v, p);
    int64_t idx = (int64_t)r * cols + c;
    switch (v->w_type) {
        case ORC_W_F32: {
            float f;
            memcpy(&f, v->w[p] + 4 * idx, 4);
            return f;
        }
        case ORC_W_BF16: {
            uint16_t h;
            memcpy(&h, v->w[p] + 2 * idx, 2);
            return bf16_value(h);
        }
        case ORC_W_W8A8:
            return (float)(int8_t)v->w[p][idx] * row_scale_i8(v, p, r);
        default: {
            int blk = c / 32, j = c % 32;
            uint8_t byte = v->w[p][(int64_t)r * (cols / 2) + 16 * blk + (j % 16)];
            int q = j < 16 ? (byte & 0xF) : (byte >> 4);
            uint16_t dh;
            memcpy(&dh, v->s[p] + 2 * ((int64_t)r * (cols / 32) + blk), 2);
            return half_value(dh) * (float)(q - 8);
        }
    }
}

int oracle_decode_expert(int w_type, const uint8_t* slab, int H, int I, float* wg, float* wu, float* wd) {
    if (w_type < 0 || w_type > 3) return -1;
    expert_view v;
    view_expert(&v, w_type, slab, H, I);
    float* dst[3] = {wg, wu, wd};
    for (int p = 0; p < 3; ++p) {
        int rows = p == 2 ? H : I, cols = proj_cols(&v, p);
        for (int r = 0; r < rows; ++r)
            for (int c = 0; c < cols; ++c) dst[p][(int64_t)r * cols + c] = weight(&v, p, r, c);
    }
    return 0;
}

static double x_value(const void* x, int x_dtype, int64_t i) {
    if (x_dtype == ORC_X_F32) return ((const float*)x)[i];
    return bf16_value(((const uint16_t*)x)[i]);
}

/* ------------------------------------------------------------ routing */

/* Router logits.  [PGO] "The method in five lines" picks top-k by the
 * router's logit; the logit is the plain product of the token with the gate
 * matrix G[E][H] (one row per expert, like every weight stored [out][in]),
 * summed in double and rounded once to fp32. */
int oracle_logits(const void* x, int x_dtype, const void* G, int T, int H, int E, float* z) {
    if (T < 0 || H <= 0 || E <= 0) return -1;
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += x_value(x, x_dtype, (int64_t)t * H + h) * x_value(G, x_dtype, (int64_t)e * H + h);
            z[(int64_t)t * E + e] = (float)acc;
        }
    return 0;
}

/* Graded bias, [PGO] "The method in five lines": experts of the hot set get
 * no penalty; every other expert gets max(cap, ln(b / b_edge)), where b_edge
 * is the brightness of the weakest hot expert.  The hot set is read as the
 * n_hot brightest experts, ties to the lower id.  b = 0 gives ln 0 = -inf,
 * so the cap.  Computed in double, stored as fp32. */
int oracle_bias_table(const double* b, int E, int n_hot, float cap, float* bias) {
    if (E <= 0 || n_hot < 1) return -1;
    if (n_hot >= E) {
        for (int e = 0; e < E; ++e) bias[e] = 0.0f;
        return 0;
    }
    /* rank of e = number of experts brighter than e, or equally bright with a lower id */
    int edge = -1;
    unsigned char* hot = (unsigned char*)calloc((size_t)E, 1);
    if (!hot) return -2;
    for (int e = 0; e < E; ++e) {
        int rank = 0;
        for (int o = 0; o < E; ++o)
            if (b[o] > b[e] || (b[o] == b[e] && o < e)) ++rank;
        if (rank < n_hot) hot[e] = 1;
        if (rank == n_hot - 1) edge = e;
    }
    double b_edge = b[edge];
    for (int e = 0; e < E; ++e) {
        if (hot[e]) { bias[e] = 0.0f; continue; }
        double v = (b[e] > 0.0 && b_edge > 0.0) ? log(b[e] / b_edge) : -INFINITY;
        bias[e] = (float)(v > (double)cap ? v : (double)cap);
    }
    free(hot);
    return 0;
}

/* Top-k by logit + bias, [PGO] "The method in five lines".  The score is one
 * fp32 add; the k best are taken one at a time (higher score first, then the
 * lower expert id) and listed in that order.  Scores must be free of NaN (the
 * callers' inputs are finite): a NaN never compares greater, so its rank here
 * would depend on where it sits rather than follow any order. */
int oracle_topk(const float* z, const float* bias, int T, int E, int k, int32_t* ids) {
    if (k < 1 || k > E) return -1;
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!s || !taken) { free(s); free(taken); return -2; }
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            float v = z[(int64_t)t * E + e];
            if (bias) v = v + bias[e];
            s[e] = v;
            taken[e] = 0;
        }
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || s[e] > s[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
    }
    free(s); free(taken);
    return 0;
}

/* Routing weights, [PGO] "The method in five lines" ("router's own softmax
 * over the picked k", selection-only): the softmax of the raw (unbiased)
 * logits restricted to the k picked experts, in double, stored as fp32. */
int oracle_route_weights(const float* z, const int32_t* ids, int T, int E, int k, float* w) {
    if (k < 1) return -1;
    for (int t = 0; t < T; ++t) {
        const int32_t* id = ids + (int64_t)t * k;
        for (int j = 0; j < k; ++j)
            if (id[j] < 0 || id[j] >= E) return -1;
        double m = -INFINITY;
        for (int j = 0; j < k; ++j) {
            double v = z[(int64_t)t * E + id[j]];
            if (v > m) m = v;
        }
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp((double)z[(int64_t)t * E + id[j]] - m);
        for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(exp((double)z[(int64_t)t * E + id[j]] - m) / sum);
    }
    return 0;
}

/* Flat soft bias and hard mask, [PGO] "Experts that don't fit": the hot set
 * (the same n_hot brightest experts as the graded table, ties to the lower
 * id) gets 0, every other expert the one number `value`; value = -inf is the
 * hard mask (a cold expert can never beat a hot one). */
int oracle_bias_flat(const double* b, int E, int n_hot, float value, float* bias) {
    if (E <= 0 || n_hot < 1 || value != value || value > 0.0f) return -1;
    for (int e = 0; e < E; ++e) {
        int rank = 0;
        for (int o = 0; o < E; ++o)
            if (b[o] > b[e] || (b[o] == b[e] && o < e)) ++rank;
        bias[e] = rank < n_hot ? 0.0f : value;
    }
    return 0;
}

/* Live-cache affinity, [PGO] "Then Maya's own knob beat ours": every expert
 * that is in VRAM right now (e2s[e] >= 0 in the cache state) has lambda added
 * to its selection score; on top of an optional static table, one fp32 add. */
int oracle_bias_affinity(const int32_t* e2s, const float* base, int E, float lambda, float* bias) {
    if (E <= 0 || !(lambda - lambda == 0.0f)) return -1;
    for (int e = 0; e < E; ++e) {
        float v = base ? base[e] : 0.0f;
        if (e2s[e] >= 0) v = v + lambda;
        bias[e] = v;
    }
    return 0;
}

/* Damped weights, [PGO] "Qwen on Strata: the bias as a quality dial": the
 * alternative to selection-only in which the weights are the softmax of the
 * biased scores s = fl32(z + bias) over the picked k, in double, as fp32. */
int oracle_route_weights_damped(const float* z, const float* bias, const int32_t* ids, int T, int E, int k, float* w) {
    if (k < 1) return -1;
    for (int t = 0; t < T; ++t) {
        const int32_t* id = ids + (int64_t)t * k;
        double s[64];
        if (k > 64) return -1;
        for (int j = 0; j < k; ++j) {
            if (id[j] < 0 || id[j] >= E) return -1;
            float v = z[(int64_t)t * E + id[j]];
            if (bias) v = v + bias[id[j]];
            s[j] = v;
        }
        double m = -INFINITY;
        for (int j = 0; j < k; ++j)
            if (s[j] > m) m = s[j];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp(s[j] - m);
        for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(exp(s[j] - m) / sum);
    }
    return 0;
}

/* -------------------------------------------------------- expert FFN */

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Symmetric int8 quantisation of a vector (per token for x, per pair for h):
 * scale = absmax / 127 (1 if the vector is all zero), code =
 * clamp(rint(v / scale), -127, 127).  Done in fp32, the precision the GPU
 * kernel takes the same decision in. */
static float quant_i8(const float* v, int n, int8_t* q) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float s = amax > 0.0f ? amax / 127.0f : 1.0f;
    for (int i = 0; i < n; ++i) {
        float c = rintf(v[i] / s);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        q[i] = (int8_t)c;
    }
    return s;
}

/* SwiGLU expert (the configurations' "SwiGLU (gate/up/down)"):
 * o = Wd (silu(Wg x) * (Wu x)).  Per-format rules:
 *  - fp32: all in double.
 *  - bf16 and 4-bit: dots in double; h is rounded to fp32 then to bf16 before
 *    the down projection.
 *  - W8A8: x and h are quantised to int8 (see quant_i8); integer dots are
 *    exact; dequantisation is ((float)acc * s_act) * s_row in fp32; h is
 *    silu(g) * u in double rounded to fp32 before it is quantised. */
int oracle_expert(int w_type, const uint8_t* slab, int H, int I, const void* x_row, int x_dtype, double* o) {
    if (w_type < 0 || w_type > 3 || H <= 0 || I <= 0) return -1;
    expert_view v;
    view_expert(&v, w_type, slab, H, I);
    if (w_type == ORC_W_W8A8) {
        float* xf = (float*)malloc(sizeof(float) * (size_t)H);
        float* h = (float*)malloc(sizeof(float) * (size_t)I);
        int8_t* qx = (int8_t*)malloc((size_t)H);
        int8_t* qh = (int8_t*)malloc((size_t)I);
        if (!xf || !h || !qx || !qh) { free(xf); free(h); free(qx); free(qh); return -2; }
        for (int i = 0; i < H; ++i) xf[i] = (float)x_value(x_row, x_dtype, i);
        float sx = quant_i8(xf, H, qx);
        for (int n = 0; n < I; ++n) {
            int64_t ag = 0, au = 0;
            for (int i = 0; i < H; ++i) {
                ag += (int64_t)qx[i] * (int8_t)v.w[0][(int64_t)n * H + i];
                au += (int64_t)qx[i] * (int8_t)v.w[1][(int64_t)n * H + i];
            }
            float g = ((float)ag * sx) * row_scale_i8(&v, 0, n);
            float u = ((float)au * sx) * row_scale_i8(&v, 1, n);
            h[n] = (float)(silu((double)g) * (double)u);
        }
        float sh = quant_i8(h, I, qh);
        for (int m = 0; m < H; ++m) {
            int64_t ad = 0;
            for (int n = 0; n < I; ++n) ad += (int64_t)qh[n] * (int8_t)v.w[2][(int64_t)m * I + n];
            o[m] = (double)(((float)ad * sh) * row_scale_i8(&v, 2, m));
        }
        free(xf); free(h); free(qx); free(qh);
        return 0;
    }
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!h) return -2;
    for (int n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int i = 0; i < H; ++i) {
            double xi = x_value(x_row, x_dtype, i);
            g += (double)weight(&v, 0, n, i) * xi;
            u += (double)weight(&v, 1, n, i) * xi;
        }
        double hv = silu(g) * u;
        if (w_type != ORC_W_F32) hv = (double)round_bf16((float)hv);
        h[n] = hv;
    }
    for (int m = 0; m < H; ++m) {
        double acc = 0.0;
        for (int n = 0; n < I; ++n) acc += (double)weight(&v, 2, m, n) * h[n];
        o[m] = acc;
    }
    free(h);
    return 0;
}

/* Whole layer.  y_full[t] = sum over the k picks of w_tj * expert(x_t), in
 * top-k order, in double.  The split follows [RTX] "What the video covers"
 * and the transcript's zero-return design: picks whose slot is >= 0 go to
 * y_gpu, the others (experts not resident) to y_host; y_gpu + y_host is the
 * full layer.  slot_ids may be NULL (no split; y_gpu / y_host untouched). */
int oracle_layer(int w_type, const uint8_t* store, int64_t slab_bytes, int E, int H, int I, const void* x,
                 int x_dtype, const int32_t* ids, const int32_t* slot_ids, const float* w, int T, int k,
                 float* y_full, float* y_gpu, float* y_host) {
    if (slab_bytes < oracle_slab_bytes(w_type, H, I)) return -1;
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* yf = (double*)malloc(sizeof(double) * (size_t)H);
    double* yg = (double*)malloc(sizeof(double) * (size_t)H);
    double* yh = (double*)malloc(sizeof(double) * (size_t)H);
    if (!o || !yf || !yg || !yh) { free(o); free(yf); free(yg); free(yh); return -2; }
    size_t xs = x_dtype == ORC_X_F32 ? 4 : 2;
    int rc = 0;
    for (int t = 0; t < T && rc == 0; ++t) {
        for (int m = 0; m < H; ++m) yf[m] = yg[m] = yh[m] = 0.0;
        const void* xr = (const uint8_t*)x + (size_t)t * H * xs;
        for (int j = 0; j < k; ++j) {
            int e = ids[(int64_t)t * k + j];
            if (e < 0 || e >= E) { rc = -3; break; }
            rc = oracle_expert(w_type, store + (int64_t)e * slab_bytes, H, I, xr, x_dtype, o);
            if (rc) break;
            double wt = w[(int64_t)t * k + j];
            int resident = slot_ids ? slot_ids[(int64_t)t * k + j] >= 0 : 1;
            for (int m = 0; m < H; ++m) {
                double c = wt * o[m];
                yf[m] += c;
                if (resident) yg[m] += c;
                else yh[m] += c;
            }
        }
        for (int m = 0; m < H; ++m) {
            if (y_full) y_full[(int64_t)t * H + m] = (float)yf[m];
            if (slot_ids && y_gpu) y_gpu[(int64_t)t * H + m] = (float)yg[m];
            if (slot_ids && y_host) y_host[(int64_t)t * H + m] = (float)yh[m];
        }
    }
    free(o); free(yf); free(yg); free(yh);
    return rc;
}

/* ------------------------------------------------------ cache manage */

/* Victim order of slot a before slot b: empty slots first (lower slot
 * first); then LRU by last use (older first), LFU by use count then last
 * use; remaining ties to the lower slot. */
static int victim_before(int policy, const int32_t* s2e, const uint32_t* last, const uint32_t* freq, int a, int b) {
    int ea = s2e[a] >= 0, eb = s2e[b] >= 0;
    if (ea != eb) return !ea;
    if (ea) {
        if (policy == ORC_LFU && freq[a] != freq[b]) return freq[a] < freq[b];
        if (last[a] != last[b]) return last[a] < last[b];
    }
    return a < b;
}

/* One step of the slot cache, [VEC] "What this package does": the manager
 * picks victims among slots this step does not need and emits a miss list;
 * routing ids are then remapped to slot space.  Readings of what the page
 * leaves open:
 *  - needed = the distinct experts among the step's routing ids;
 *  - a hit refreshes its slot (last = step; LFU also counts one use per step);
 *  - misses are the needed, non-resident experts in ascending id; the i-th
 *    miss takes the i-th victim in victim_before order; the evicted expert
 *    leaves the map, the new one enters with last = step, freq = 1;
 *  - misses beyond the victims ("Measuring, without fooling yourself": a
 *    step is only fully served from slots when it fits) go to the host list;
 *  - STATIC never changes the map: every non-resident needed expert is a
 *    host miss;
 *  - slot_ids[i] = the slot of ids[i] after the step, -1 if not resident;
 *  - step advances by one per call.
 * stats (may be NULL): routing ids resident at entry, distinct needed,
 * gathered, host misses. */
int oracle_manage(int policy, int E, int S, int32_t* e2s, int32_t* s2e, uint32_t* last, uint32_t* freq,
                  uint32_t* step, const int32_t* ids, int n_ids, int32_t* slot_ids, int32_t* miss, int32_t* n_miss,
                  int32_t* host_miss, int32_t* n_host, int32_t* stats) {
    if (E <= 0 || S < 0 || S > E || n_ids < 0 || policy < 0 || policy > 2) return -1;
    for (int i = 0; i < n_ids; ++i)
        if (ids[i] < 0 || ids[i] >= E) return -1;
    unsigned char* need = (unsigned char*)calloc((size_t)E, 1);
    int* cand = (int*)malloc(sizeof(int) * (size_t)(S > 0 ? S : 1));
    int* misses = (int*)malloc(sizeof(int) * (size_t)E);
    if (!need || !cand || !misses) { free(need); free(cand); free(misses); return -2; }
    uint32_t now = *step;
    int hit_ids = 0, distinct = 0, nm = 0, nh = 0, ncand = 0, nmiss_all = 0;
    for (int i = 0; i < n_ids; ++i) {
        if (e2s[ids[i]] >= 0) ++hit_ids;
        need[ids[i]] = 1;
    }
    for (int e = 0; e < E; ++e) {
        if (!need[e]) continue;
        ++distinct;
        if (e2s[e] < 0) misses[nmiss_all++] = e;
        else if (policy != ORC_STATIC) {
            int s = e2s[e];
            last[s] = now;
            if (policy == ORC_LFU) freq[s] += 1;
        }
    }
    if (policy != ORC_STATIC) {
        for (int s = 0; s < S; ++s)
            if (s2e[s] < 0 || !need[s2e[s]]) cand[ncand++] = s;
        /* order the candidates (insertion sort: plain and stable) */
        for (int i = 1; i < ncand; ++i) {
            int c = cand[i], j = i - 1;
            while (j >= 0 && victim_before(policy, s2e, last, freq, c, cand[j])) {
                cand[j + 1] = cand[j];
                --j;
            }
            cand[j + 1] = c;
        }
        for (int i = 0; i < nmiss_all; ++i) {
            int e = misses[i];
            if (i < ncand) {
                int s = cand[i];
                if (s2e[s] >= 0) e2s[s2e[s]] = -1;
                s2e[s] = e;
                e2s[e] = s;
                last[s] = now;
                freq[s] = 1;
                miss[2 * nm] = e;
                miss[2 * nm + 1] = s;
                ++nm;
            } else {
                host_miss[nh++] = e;
            }
        }
    } else {
        for (int i = 0; i < nmiss_all; ++i) host_miss[nh++] = misses[i];
    }
    for (int i = 0; i < n_ids; ++i) slot_ids[i] = e2s[ids[i]];
    *n_miss = nm;
    *n_host = nh;
    *step = now + 1;
    if (stats) {
        stats[0] = hit_ids;
        stats[1] = distinct;
        stats[2] = nm;
        stats[3] = nh;
    }
    free(need); free(cand); free(misses);
    return 0;
}

/* [VEC] "What this package does": the gather copies the missing experts
 * host-to-slot; "Prove it is correct before measuring" checks that gathered
 * bytes equal their source rows. */
int oracle_gather(const int32_t* miss, int n_miss, const uint8_t* host_store, uint8_t* slot_store,
                  int64_t slab_bytes) {
    for (int i = 0; i < n_miss; ++i)
        memcpy(slot_store + (int64_t)miss[2 * i + 1] * slab_bytes, host_store + (int64_t)miss[2 * i] * slab_bytes,
               (size_t)slab_bytes);
    return 0;
}

/* Residual join of stacked layers ([PGO] "Experts that don't fit": the
 * routed layers follow one another; each adds its output to what it read).
 * The stream keeps its storage format: bf16 streams get the fp32 sum
 * rounded to bf16 (nearest, ties to even), fp32 streams the fp32 sum. */
int oracle_residual(const void* x, int x_dtype, const float* y, int T, int H, void* out) {
    const int64_t n = (int64_t)T * H;
    for (int64_t i = 0; i < n; ++i) {
        if (x_dtype == ORC_X_BF16) {
            const float v = round_bf16(bf16_value(((const uint16_t*)x)[i]) + y[i]);
            uint32_t b;
            memcpy(&b, &v, 4);
            ((uint16_t*)out)[i] = (uint16_t)(b >> 16);
        } else {
            ((float*)out)[i] = ((const float*)x)[i] + y[i];
        }
    }
    return 0;
}

/* Periodic repick, [RTX] "Full Transcript" (have another look every ~500
 * tokens, swap out whatever has gone cold, then leave the set alone): the new
 * set is the distinct valid experts of want[0..S) (a repeated or out-of-range
 * entry is skipped).  Members of the new set that are resident keep their
 * slots; the others are loaded, in ascending expert id, into the slots whose
 * expert left the set (empty slots included), in ascending slot order; a
 * slot not needed for a load keeps its expert.  miss[] lists the loads as
 * (expert, slot) pairs for the gather; a loaded slot restarts with
 * last = step, freq = 0.  step does not advance. */
int oracle_repick(int E, int S, int32_t* e2s, int32_t* s2e, uint32_t* last, uint32_t* freq,
                  const uint32_t* step, const int32_t* want, int32_t* miss, int32_t* n_miss) {
    if (E <= 0 || S < 0 || S > E) return -1;
    unsigned char* in_new = (unsigned char*)calloc((size_t)E, 1);
    if (!in_new) return -2;
    for (int i = 0; i < S; ++i)
        if (want[i] >= 0 && want[i] < E) in_new[want[i]] = 1;
    int nm = 0, s = 0;
    for (int e = 0; e < E; ++e) {
        if (!in_new[e] || e2s[e] >= 0) continue;
        /* next slot whose expert is not in the new set */
        while (s < S && s2e[s] >= 0 && in_new[s2e[s]]) ++s;
        if (s >= S) break; /* cannot happen: there are at most S members */
        if (s2e[s] >= 0) e2s[s2e[s]] = -1;
        s2e[s] = e;
        e2s[e] = s;
        last[s] = *step;
        freq[s] = 0;
        miss[2 * nm] = e;
        miss[2 * nm + 1] = s;
        ++nm;
        ++s;
    }
    *n_miss = nm;
    free(in_new);
    return 0;
}

/* Static resident set ([RTX] transcript: the set is chosen once before the
 * run from a profile of what the router picks, then never changes): count
 * picks per expert over a profile batch and keep the S most picked, ties to
 * the lower id; slot i holds the i-th of them. */
int oracle_pick_static(const int32_t* ids, int n_ids, int E, int S, int32_t* resident) {
    if (S < 0 || S > E) return -1;
    int* cnt = (int*)calloc((size_t)E, sizeof(int));
    if (!cnt) return -2;
    for (int i = 0; i < n_ids; ++i) {
        if (ids[i] < 0 || ids[i] >= E) { free(cnt); return -1; }
        cnt[ids[i]]++;
    }
    for (int e = 0; e < E; ++e) {
        int rank = 0;
        for (int o = 0; o < E; ++o)
            if (cnt[o] > cnt[e] || (cnt[o] == cnt[e] && o < e)) ++rank;
        if (rank < S) resident[rank] = e;
    }
    free(cnt);
    return 0;
}

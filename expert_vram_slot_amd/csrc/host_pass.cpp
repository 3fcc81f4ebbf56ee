// Host pass of the expert-slot layer: the SwiGLU FFN of the picks whose
// expert is not resident, on CPU threads, reading the host expert store.
//
// sozai.app transcript "rtx-3060-run-35b-llamacpp", "What the video covers"
// and "Full Transcript": the experts that stay in RAM are run by the CPU in a
// pass of their own, concurrently with the GPU pass, and one add joins the
// two results.  The arithmetic per weight format is the GPU kernels' (see
// moe_slot.h); every output element is produced by one work item in a fixed
// order, so the result does not depend on the thread count.
#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/moe_slot.h"

int moe_fail(int code, const char* fmt, ...);
int moe_ok();
int moe_layout(int w_type, int H, int I, moe_slab_layout_t* out);

namespace {

// ----------------------------------------------------------- thread pool

class Pool {
   public:
    // Run fn(item) for item in [0, n) on `threads` threads (the caller
    // included).  Items are handed out dynamically; each runs exactly once.
    // Idle workers spin for up to kSpinNs before they sleep, so the phases of
    // one call, and calls that follow each other closely (the layers of a
    // decode step, with only the GPU router between them), start without a
    // wake-up delay.
    void run(int threads, int n, const std::function<void(int)>& fn) {
        if (n <= 0) return;
        threads = std::max(1, std::min({threads, n, 64}));
        if (threads == 1) {
            for (int i = 0; i < n; ++i) fn(i);
            return;
        }
        std::lock_guard<std::mutex> serial(call_mu_);  // one call at a time
        while ((int)workers_.size() < threads - 1) {
            const int id = (int)workers_.size();
            workers_.emplace_back([this, id] { loop(id); });
        }
        {
            std::lock_guard<std::mutex> lk(mu_);
            fn_ = &fn;
            n_ = n;
            next_.store(0, std::memory_order_relaxed);
            pending_.store(threads - 1, std::memory_order_relaxed);
            // generation and the number of workers taking part, published together
            word_.store(((word_.load(std::memory_order_relaxed) >> 8) + 1) << 8 | (uint64_t)(threads - 1),
                        std::memory_order_release);
        }
        cv_.notify_all();
        work();
        for (Spin sp; pending_.load(std::memory_order_acquire) != 0 && sp.more();) _mm_pause();
        if (pending_.load(std::memory_order_acquire) != 0) {
            std::unique_lock<std::mutex> lk(mu_);
            done_cv_.wait(lk, [&] { return pending_.load(std::memory_order_acquire) == 0; });
        }
        fn_ = nullptr;
    }

    ~Pool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_.store(true);
            word_.fetch_add(1 << 8);
        }
        cv_.notify_all();
        for (auto& t : workers_) t.join();
    }

   private:
    static constexpr int64_t kSpinNs = 250000;

    // spin budget: true until kSpinNs have passed (the clock is read every 64 calls)
    struct Spin {
        std::chrono::steady_clock::time_point t0 = std::chrono::steady_clock::now();
        int n = 0;
        bool more() {
            if (++n & 63) return true;
            return std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count() <
                   kSpinNs;
        }
    };

    void work() {
        for (;;) {
            const int i = next_.fetch_add(1);
            if (i >= n_) break;
            (*fn_)(i);
        }
    }
    void loop(int id) {
        uint64_t seen = 0;
        for (;;) {
            uint64_t w = word_.load(std::memory_order_acquire);
            for (Spin sp; (w >> 8) == (seen >> 8) && sp.more();) {
                _mm_pause();
                w = word_.load(std::memory_order_acquire);
            }
            if ((w >> 8) == (seen >> 8)) {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_.load() || (word_.load() >> 8) != (seen >> 8); });
                w = word_.load(std::memory_order_acquire);
            }
            if (stop_.load()) return;
            seen = w;
            if (id >= (int)(w & 0xFF)) continue;  // not taking part in this call
            work();
            if (pending_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
                std::lock_guard<std::mutex> lk(mu_);
                done_cv_.notify_all();
            }
        }
    }

    std::mutex call_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> workers_;
    const std::function<void(int)>* fn_ = nullptr;
    std::atomic<int> next_{0};
    std::atomic<int> pending_{0};
    std::atomic<uint64_t> word_{0};  // generation << 8 | workers taking part
    std::atomic<bool> stop_{false};
    int n_ = 0;
};

Pool& pool() {
    static Pool p;
    return p;
}

void parallel(int threads, int n, const std::function<void(int)>& fn) { pool().run(threads, n, fn); }

// ---------------------------------------------------------- scratch

// Intermediate rows of the pass, kept per calling thread between calls so
// that a step neither zero-fills nor faults in its buffers again: every
// element the pass reads it has written in the same call (the rows of the
// picks it serves).  A buffer above KEEP_BYTES is released when its call
// ends, so only decode-sized needs stay allocated.
constexpr size_t KEEP_BYTES = size_t(64) << 20;
enum ScratchBuf { SB_XF, SB_XQ, SB_XS, SB_XW, SB_XBS, SB_XP, SB_HF, SB_HQ, SB_HS, SB_HW, SB_HB, SB_HBS, SB_HP, SB_PART,
                  SB_COUNT };

struct Scratch {
    void* p[SB_COUNT] = {};
    size_t cap[SB_COUNT] = {};
    ~Scratch() {
        for (void* q : p) free(q);
    }
};
thread_local Scratch tl_scratch;

// n elements of buffer b, 64-byte aligned, contents undefined; nullptr when
// the allocation fails (n == 0 gives a valid pointer too)
template <class T>
T* scratch(ScratchBuf b, size_t n) {
    Scratch& s = tl_scratch;
    const size_t bytes = (std::max<size_t>(n * sizeof(T), 64) + 63) & ~size_t(63);
    if (bytes > s.cap[b]) {
        free(s.p[b]);
        s.p[b] = aligned_alloc(64, bytes);
        s.cap[b] = s.p[b] ? bytes : 0;
    }
    return static_cast<T*>(s.p[b]);
}

// releases the call's buffers above KEEP_BYTES on every return path
struct ScratchTrim {
    ~ScratchTrim() {
        Scratch& s = tl_scratch;
        for (int b = 0; b < SB_COUNT; ++b)
            if (s.cap[b] > KEEP_BYTES) {
                free(s.p[b]);
                s.p[b] = nullptr;
                s.cap[b] = 0;
            }
    }
};

// ---------------------------------------------------------- formats

inline float bf16f(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

inline uint16_t f2bf(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

inline float half_to_float(uint16_t h) { return _cvtsh_ss(h); }

// one bf16 weight row against NT <= 4 bf16 activation rows, n % 32 == 0:
// the row is loaded once per 32 inputs for all NT rows, and each activation
// row keeps four accumulators (32-input chunk j goes to accumulator j mod 4),
// so a row's sum runs in the same order whatever NT is
template <int NT>
__attribute__((target("avx512f,avx512bf16"))) void dot_bf16x(const uint16_t* w, const uint16_t* const* x, int n,
                                                              float* out) {
    __m512 acc[NT][4];
    for (int t = 0; t < NT; ++t)
        for (int a = 0; a < 4; ++a) acc[t][a] = _mm512_setzero_ps();
    int i = 0;
    for (; i + 128 <= n; i += 128) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const __m512i wv = _mm512_loadu_si512(reinterpret_cast<const void*>(w + i + 32 * a));
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t][a] = _mm512_dpbf16_ps(acc[t][a], (__m512bh)wv,
                                             (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i + 32 * a)));
        }
    }
    for (int a = 0; i < n; i += 32, ++a) {
        const __m512i wv = _mm512_loadu_si512(reinterpret_cast<const void*>(w + i));
        for (int t = 0; t < NT; ++t)
            acc[t][a] = _mm512_dpbf16_ps(acc[t][a], (__m512bh)wv,
                                         (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i)));
    }
    for (int t = 0; t < NT; ++t)
        out[t] = _mm512_reduce_add_ps(_mm512_add_ps(_mm512_add_ps(acc[t][0], acc[t][1]), _mm512_add_ps(acc[t][2], acc[t][3])));
}

void dot_bf16x_rows(int nt, const uint16_t* w, const uint16_t* const* x, int n, float* out) {
    switch (nt) {
        case 1: dot_bf16x<1>(w, x, n, out); break;
        case 2: dot_bf16x<2>(w, x, n, out); break;
        case 3: dot_bf16x<3>(w, x, n, out); break;
        default: dot_bf16x<4>(w, x, n, out); break;
    }
}

float dot_bf16_plain(const uint16_t* w, const uint16_t* x, int n) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < n; i += 8)
        for (int j = 0; j < 8; ++j) acc[j] += bf16f(w[i + j]) * bf16f(x[i + j]);
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

bool have_avx512bf16() {
    static const bool v = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bf16");
    return v;
}

float dot_f32(const float* w, const float* x, int n) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int i = 0;
    for (; i + 8 <= n; i += 8)
        for (int j = 0; j < 8; ++j) acc[j] += w[i + j] * x[i + j];
    float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    for (; i < n; ++i) s += w[i] * x[i];
    return s;
}

int32_t dot_i8(const int8_t* w, const int8_t* x, int n) {
    int32_t acc = 0;
    for (int i = 0; i < n; ++i) acc += (int32_t)w[i] * (int32_t)x[i];
    return acc;
}

// one int8 weight row against NT <= 4 int8 activation rows held widened to
// int16, n % 32 == 0: the row is widened once per 32 inputs for all NT rows;
// exact int32 sums, so the grouping cannot change a result
template <int NT>
__attribute__((target("avx512f,avx512bw"))) void dot_i8x(const int8_t* w, const int16_t* const* x, int n,
                                                          int32_t* out) {
    __m512i acc[NT][2];
    for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = _mm512_setzero_si512();
    int i = 0;
    for (; i + 64 <= n; i += 64) {
        const __m512i w0 = _mm512_cvtepi8_epi16(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i)));
        const __m512i w1 = _mm512_cvtepi8_epi16(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i + 32)));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t][0] = _mm512_add_epi32(
                acc[t][0], _mm512_madd_epi16(w0, _mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i))));
            acc[t][1] = _mm512_add_epi32(
                acc[t][1], _mm512_madd_epi16(w1, _mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i + 32))));
        }
    }
    if (i < n) {
        const __m512i w0 = _mm512_cvtepi8_epi16(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i)));
        for (int t = 0; t < NT; ++t)
            acc[t][0] = _mm512_add_epi32(
                acc[t][0], _mm512_madd_epi16(w0, _mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i))));
    }
    for (int t = 0; t < NT; ++t) out[t] = _mm512_reduce_add_epi32(_mm512_add_epi32(acc[t][0], acc[t][1]));
}

void dot_i8x_rows(int nt, const int8_t* w, const int16_t* const* x, int n, int32_t* out) {
    switch (nt) {
        case 1: dot_i8x<1>(w, x, n, out); break;
        case 2: dot_i8x<2>(w, x, n, out); break;
        case 3: dot_i8x<3>(w, x, n, out); break;
        default: dot_i8x<4>(w, x, n, out); break;
    }
}

// The same rows with AVX-512 VNNI, the activations held as u8 = x + 128 (n % 64
// == 0): dpbusd adds four u8 x s8 products into each int32 lane, so the row
// gives sum (x + 128) w = sum x w + 128 sum w, and one more dpbusd against
// ones (the row's sum of w, shared by the NT rows) takes the offset out.  All
// of it is exact modulo 2^32 (unsigned at the end), and the result, at most
// 127 * 128 * n in magnitude, fits int32, so it is the one the int16 path gives.
template <int NT>
__attribute__((target("avx512f,avx512bw,avx512vnni"))) void dot_i8u(const int8_t* w, const uint8_t* const* x, int n,
                                                                     int32_t* out) {
    __m512i acc[NT];
    __m512i sw = _mm512_setzero_si512();
    const __m512i ones = _mm512_set1_epi8(1);
    for (int t = 0; t < NT; ++t) acc[t] = _mm512_setzero_si512();
    for (int i = 0; i < n; i += 64) {
        const __m512i wv = _mm512_loadu_si512(reinterpret_cast<const void*>(w + i));
        sw = _mm512_dpbusd_epi32(sw, ones, wv);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = _mm512_dpbusd_epi32(acc[t], _mm512_loadu_si512(reinterpret_cast<const void*>(x[t] + i)), wv);
    }
    const uint32_t s = (uint32_t)_mm512_reduce_add_epi32(sw);
    for (int t = 0; t < NT; ++t) out[t] = (int32_t)((uint32_t)_mm512_reduce_add_epi32(acc[t]) - 128u * s);
}

void dot_i8u_rows(int nt, const int8_t* w, const uint8_t* const* x, int n, int32_t* out) {
    switch (nt) {
        case 1: dot_i8u<1>(w, x, n, out); break;
        case 2: dot_i8u<2>(w, x, n, out); break;
        case 3: dot_i8u<3>(w, x, n, out); break;
        default: dot_i8u<4>(w, x, n, out); break;
    }
}

// one int8 row against nt activation rows in the form the pass keeps them:
// u8 = x + 128 (vnni) or int16
void dot_i8_rows(bool vnni, int nt, const int8_t* w, const void* const* x, int n, int32_t* out) {
    if (vnni) dot_i8u_rows(nt, w, reinterpret_cast<const uint8_t* const*>(x), n, out);
    else dot_i8x_rows(nt, w, reinterpret_cast<const int16_t* const*>(x), n, out);
}

bool have_avx512bw() {
    static const bool v = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
    return v;
}

bool have_avx512vnni() {
    static const bool v = have_avx512bw() && __builtin_cpu_supports("avx512vnni");
    return v;
}

bool have_avx512vl() {
    static const bool v = __builtin_cpu_supports("avx512vl");
    return v;
}

// 4-bit row (nibble plane row + fp16 scales) against fp32 activations
float dot_q4(const uint8_t* q, const uint16_t* sc, const float* x, int n) {
    float acc = 0.0f;
    for (int b = 0; b < n / 32; ++b) {
        const uint8_t* blk = q + 16 * b;
        const float* xb = x + 32 * b;
        float d = 0.0f;
        for (int j = 0; j < 16; ++j) {
            d += (float)((int)(blk[j] & 0xF) - 8) * xb[j];
            d += (float)((int)(blk[j] >> 4) - 8) * xb[j + 16];
        }
        acc += half_to_float(sc[b]) * d;
    }
    return acc;
}

// 4-bit row against bf16 activations with AVX-512 BF16: each code q is put in
// the mantissa of 0x4300 (the bf16 value 128 + q, exact), one dpbf16 gives
// sum (q + 128) x over a 32-weight block, and the block's sum of x removes
// the offset: sum (q - 8) x = sum (q + 128) x - 136 sum x.  Low nibbles are
// inputs 0..15 of a block, high nibbles 16..31.  xsum: per-block sums of x.
// one 32-weight block: acc += s * dpbf16(128 + q, x)
__attribute__((target("avx512f,avx512bw,avx512bf16"), always_inline)) inline void q4_block(const uint8_t* q,
                                                                                           const uint16_t* xb,
                                                                                           float s, __m512& acc) {
    const __m128i m4 = _mm_set1_epi8(0x0F);
    const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(q));
    const __m128i lo = _mm_and_si128(v, m4);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(v, 4), m4);
    const __m512i w16 = _mm512_or_si512(_mm512_cvtepu8_epi16(_mm256_set_m128i(hi, lo)), _mm512_set1_epi16(0x4300));
    const __m512i xv = _mm512_loadu_si512(reinterpret_cast<const void*>(xb));
    const __m512 d = _mm512_dpbf16_ps(_mm512_setzero_ps(), (__m512bh)w16, (__m512bh)xv);
    acc = _mm512_fmadd_ps(_mm512_set1_ps(s), d, acc);
}

__attribute__((target("avx512f,avx512bw,avx512bf16,avx512vl"))) float dot_q4_avx512(const uint8_t* q,
                                                                                      const uint16_t* sc,
                                                                                      const uint16_t* xb,
                                                                                      const float* xsum, int n) {
    __m512 acc0 = _mm512_setzero_ps(), acc1 = _mm512_setzero_ps(), corr = _mm512_setzero_ps();
    const int nb = n / 32;
    int b0 = 0;
    for (; b0 + 16 <= nb; b0 += 16) {  // 16 scales at a time; the offset term as one vector FMA
        const __m512 s16 = _mm512_cvtph_ps(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(sc + b0)));
        corr = _mm512_fmadd_ps(s16, _mm512_loadu_ps(xsum + b0), corr);
        alignas(64) float sa[16];
        _mm512_store_ps(sa, s16);
        for (int j = 0; j < 16; j += 2) {
            q4_block(q + 16 * (b0 + j), xb + 32 * (b0 + j), sa[j], acc0);
            q4_block(q + 16 * (b0 + j + 1), xb + 32 * (b0 + j + 1), sa[j + 1], acc1);
        }
    }
    float tail = 0.0f;
    for (; b0 < nb; ++b0) {
        const float s = _cvtsh_ss(sc[b0]);
        q4_block(q + 16 * b0, xb + 32 * b0, s, acc0);
        tail += s * xsum[b0];
    }
    return _mm512_reduce_add_ps(_mm512_add_ps(acc0, acc1)) - 136.0f * (_mm512_reduce_add_ps(corr) + tail);
}

// The same 4-bit dot, four blocks (128 weights) per step: the 64 code bytes
// of four blocks fill one 512-bit register, one block per 128-bit lane, and
// byte interleaves with 0x43 turn the nibbles into the bf16 values 128 + q in
// place.  An interleave stays inside its 128-bit lane, so the activations are
// stored to match (q4x_order), and every fp32 lane of a product belongs to
// one block and takes that block's scale.  NT activation rows share each
// decoded group; each row's sum runs in the same order whatever NT is.
// n % 128 == 0.
void q4x_order(const uint16_t* x, int n, uint16_t* xp) {
    // group g (blocks 4g..4g+3), part c (inputs 8c..8c+7 of a block), block L, input i
    for (int g = 0; g < n / 128; ++g)
        for (int c = 0; c < 4; ++c)
            for (int L = 0; L < 4; ++L)
                for (int i = 0; i < 8; ++i) xp[128 * g + 32 * c + 8 * L + i] = x[32 * (4 * g + L) + 8 * c + i];
}

template <int NT>
__attribute__((target("avx512f,avx512bw,avx512bf16,avx512vl"))) void dot_q4x(const uint8_t* q, const uint16_t* sc,
                                                                                const uint16_t* const* xp,
                                                                                const float* const* xsum, int n,
                                                                                float* out) {
    __m512 acc[NT];
    __m128 corr[NT];
    for (int t = 0; t < NT; ++t) {
        acc[t] = _mm512_setzero_ps();
        corr[t] = _mm_setzero_ps();
    }
    const __m512i m4 = _mm512_set1_epi8(0x0F), c43 = _mm512_set1_epi8(0x43);
    const __m512i lane_block = _mm512_set_epi32(3, 3, 3, 3, 2, 2, 2, 2, 1, 1, 1, 1, 0, 0, 0, 0);
    for (int g = 0; g < n / 128; ++g) {
        const __m512i v = _mm512_loadu_si512(reinterpret_cast<const void*>(q + 64 * g));
        const __m512i lo = _mm512_and_si512(v, m4), hi = _mm512_and_si512(_mm512_srli_epi16(v, 4), m4);
        const __m512i w0 = _mm512_unpacklo_epi8(lo, c43), w1 = _mm512_unpackhi_epi8(lo, c43);
        const __m512i w2 = _mm512_unpacklo_epi8(hi, c43), w3 = _mm512_unpackhi_epi8(hi, c43);
        const __m128 s4 = _mm_cvtph_ps(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(sc + 4 * g)));
        const __m512 S = _mm512_permutexvar_ps(lane_block, _mm512_castps128_ps512(s4));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t* p = xp[t] + 128 * g;
            __m512 d = _mm512_dpbf16_ps(_mm512_setzero_ps(), (__m512bh)w0,
                                        (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(p)));
            d = _mm512_dpbf16_ps(d, (__m512bh)w1, (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(p + 32)));
            d = _mm512_dpbf16_ps(d, (__m512bh)w2, (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(p + 64)));
            d = _mm512_dpbf16_ps(d, (__m512bh)w3, (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(p + 96)));
            acc[t] = _mm512_fmadd_ps(S, d, acc[t]);
            corr[t] = _mm_fmadd_ps(s4, _mm_loadu_ps(xsum[t] + 4 * g), corr[t]);
        }
    }
    for (int t = 0; t < NT; ++t) {
        __m128 c = corr[t];
        c = _mm_add_ps(c, _mm_movehl_ps(c, c));
        c = _mm_add_ss(c, _mm_movehdup_ps(c));
        out[t] = _mm512_reduce_add_ps(acc[t]) - 136.0f * _mm_cvtss_f32(c);
    }
}

// one 4-bit row against nt <= 4 activation rows
void dot_q4x_rows(int nt, const uint8_t* q, const uint16_t* sc, const uint16_t* const* xp, const float* const* xsum,
                  int n, float* out) {
    switch (nt) {
        case 1: dot_q4x<1>(q, sc, xp, xsum, n, out); break;
        case 2: dot_q4x<2>(q, sc, xp, xsum, n, out); break;
        case 3: dot_q4x<3>(q, sc, xp, xsum, n, out); break;
        default: dot_q4x<4>(q, sc, xp, xsum, n, out); break;
    }
}

// Software prefetch of the weight row `ahead` rows past row r (each stream
// about 4 KiB ahead).  Pinned host memory comes in 4 KiB pages, and hardware
// prefetchers stop at page boundaries; a prefetch instruction does not.
struct RowPrefetch {
    const unsigned char* base;
    size_t row_bytes;
    int rows, ahead;
    RowPrefetch(const void* b, size_t rb, int n)
        : base(reinterpret_cast<const unsigned char*>(b)), row_bytes(rb), rows(n),
          ahead((int)std::max<size_t>(1, 4096 / rb)) {}
    void operator()(int r) const {
        if (r + ahead >= rows) return;
        const unsigned char* p = base + (size_t)(r + ahead) * row_bytes;
        for (size_t o = 0; o < row_bytes; o += 64) _mm_prefetch(reinterpret_cast<const char*>(p + o), _MM_HINT_T0);
    }
};

// per-block (32 inputs) sums of bf16 rows, fp32 in input order
void block_sums(const uint16_t* x, int n, float* out) {
    for (int b = 0; b < n / 32; ++b) {
        float s = 0.0f;
        for (int j = 0; j < 32; ++j) s += bf16f(x[32 * b + j]);
        out[b] = s;
    }
}

// symmetric int8 quantisation, fp32 decisions (as on the GPU)
float quant_row(const float* v, int n, int8_t* q) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) amax = std::max(amax, fabsf(v[i]));
    const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
    for (int i = 0; i < n; ++i) {
        float c = rintf(v[i] / s);
        c = std::min(std::max(c, -127.0f), 127.0f);
        q[i] = (int8_t)c;
    }
    return s;
}

}  // namespace

extern "C" int moe_ffn_host_misses(const void* x_h, int x_dtype, const int32_t* ids_h, const int32_t* slot_ids_h,
                                   const float* w_h, int T, int k, const void* host_store, size_t slab_bytes, int E,
                                   int w_type, int H, int I, float* y_h, int n_threads) {
    if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return moe_fail(MOE_E_ARG, "moe_ffn_host_misses: bad sizes");
    if (T == 0) return moe_ok();
    if (!x_h || !ids_h || !slot_ids_h || !w_h || !host_store || !y_h)
        return moe_fail(MOE_E_ARG, "moe_ffn_host_misses: NULL argument");
    moe_slab_layout_t lay;
    int rc = moe_layout(w_type, H, I, &lay);
    if (rc) return rc;
    if (slab_bytes < (size_t)lay.total)
        return moe_fail(MOE_E_ALIGN, "moe_ffn_host_misses: slab_bytes=%zu < %lld", slab_bytes, (long long)lay.total);
    const int want_x = w_type == MOE_W_F32 ? MOE_X_F32 : MOE_X_BF16;
    if (x_dtype != want_x)
        return moe_fail(MOE_E_DTYPE, "moe_ffn_host_misses: weight format %d needs activation format %d", w_type, want_x);
    if (n_threads < 1) n_threads = 1;

    const int P = T * k;
    // picks served here: slot < 0 with a valid expert, grouped by expert (pick order kept)
    std::vector<int> cnt(E + 1, 0);
    for (int p = 0; p < P; ++p)
        if (slot_ids_h[p] < 0 && ids_h[p] >= 0 && ids_h[p] < E) cnt[ids_h[p] + 1]++;
    for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
    std::vector<int> order(cnt[E]);
    {
        std::vector<int> fill(cnt.begin(), cnt.end() - 1);
        for (int p = 0; p < P; ++p)
            if (slot_ids_h[p] < 0 && ids_h[p] >= 0 && ids_h[p] < E) order[fill[ids_h[p]]++] = p;
    }
    std::vector<int> experts;
    for (int e = 0; e < E; ++e)
        if (cnt[e + 1] > cnt[e]) experts.push_back(e);
    const int NE = (int)experts.size();
    const unsigned char* store = reinterpret_cast<const unsigned char*>(host_store);

    // per-token activation forms, one token per work item: bf16 bits as given
    // (bf16, 4-bit), fp32 (fp32 as given; 4-bit scalar path and W8A8), int8
    // with its scale and widened to int16 (W8A8), and for 4-bit the block sums
    // and, with H and I in whole groups of four blocks, the grouped order
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x_h);
    const bool q4_fast = w_type == MOE_W_Q4B32 && have_avx512bf16() && have_avx512bw() && have_avx512vl();
    const bool q4x = q4_fast && H % 128 == 0 && I % 128 == 0;
    const bool i8_fast = w_type == MOE_W_W8A8 && have_avx512bw() && H % 32 == 0 && I % 32 == 0;
    const bool i8_vnni = i8_fast && have_avx512vnni() && H % 64 == 0 && I % 64 == 0;
    const bool need_xf = w_type == MOE_W_W8A8 || (w_type == MOE_W_Q4B32 && !q4_fast);
    const bool bf16_fast = w_type == MOE_W_BF16 && have_avx512bf16() && H % 32 == 0 && I % 32 == 0;
    const bool need_hb = (w_type == MOE_W_BF16 && bf16_fast) || q4_fast;
    const bool w8 = w_type == MOE_W_W8A8;
    const ScratchTrim trim;
    float* xf = scratch<float>(SB_XF, need_xf ? (size_t)T * H : 0);
    const float* xfp = w_type == MOE_W_F32 ? reinterpret_cast<const float*>(x_h) : xf;
    int8_t* xq = scratch<int8_t>(SB_XQ, w8 ? (size_t)T * H : 0);
    float* xs = scratch<float>(SB_XS, w8 ? T : 0);
    // W8A8: int8 activations as u8 = x + 128 (VNNI) or widened to int16, once
    int16_t* xw = scratch<int16_t>(SB_XW, i8_fast ? (size_t)T * H : 0);
    float* xbs = scratch<float>(SB_XBS, q4_fast ? (size_t)T * (H / 32) : 0);  // 4-bit: per-block sums of x
    uint16_t* xp = scratch<uint16_t>(SB_XP, q4x ? (size_t)T * H : 0);        // 4-bit: grouped order
    // per pick: h (fp32; bf16-rounded where the format says so), its int8
    // codes and scale and the codes widened (W8A8), its bf16 bits (bf16,
    // 4-bit), block sums and grouped order (4-bit), and w * FFN(x) rows
    float* hf = scratch<float>(SB_HF, (size_t)P * I);
    int8_t* hq = scratch<int8_t>(SB_HQ, w8 ? (size_t)P * I : 0);
    float* hs = scratch<float>(SB_HS, w8 ? P : 0);
    int16_t* hw = scratch<int16_t>(SB_HW, i8_fast ? (size_t)P * I : 0);
    uint16_t* hb = scratch<uint16_t>(SB_HB, need_hb ? (size_t)P * I : 0);
    float* hbs = scratch<float>(SB_HBS, q4_fast ? (size_t)P * (I / 32) : 0);
    uint16_t* hp = scratch<uint16_t>(SB_HP, q4x ? (size_t)P * I : 0);
    float* part = scratch<float>(SB_PART, (size_t)P * H);
    if (!xf || !xq || !xs || !xw || !xbs || !xp || !hf || !hq || !hs || !hw || !hb || !hbs || !hp || !part)
        return moe_fail(MOE_E_NOMEM, "moe_ffn_host_misses: cannot allocate %zu bytes of host scratch",
                        (size_t)P * (I * 4 + H * 4));
    const std::function<void(int)> prep_token = [&](int t) {
        const uint16_t* xr = xb + (size_t)t * H;
        if (need_xf)
            for (int i = 0; i < H; ++i) xf[(size_t)t * H + i] = bf16f(xr[i]);
        if (w_type == MOE_W_W8A8) {
            xs[t] = quant_row(&xf[(size_t)t * H], H, &xq[(size_t)t * H]);
            if (i8_vnni) {
                uint8_t* xu = reinterpret_cast<uint8_t*>(xw) + (size_t)t * H;
                for (int i = 0; i < H; ++i) xu[i] = (uint8_t)(xq[(size_t)t * H + i] + 128);
            } else if (i8_fast) {
                for (int i = 0; i < H; ++i) xw[(size_t)t * H + i] = xq[(size_t)t * H + i];
            }
        }
        if (q4_fast) block_sums(xr, H, &xbs[(size_t)t * (H / 32)]);
        if (q4x) q4x_order(xr, H, &xp[(size_t)t * H]);
    };
    if (w_type != MOE_W_F32 && w_type != MOE_W_BF16) {
        if (T >= 8) parallel(n_threads, T, prep_token);
        else
            for (int t = 0; t < T; ++t) prep_token(t);
    }

    // phase 1: gate/up rows, blocks of RB rows per work item
    const int RB = 32;
    const int nrb = (I + RB - 1) / RB;
    parallel(n_threads, NE * nrb, [&](int item) {
        const int e = experts[item / nrb], r0 = (item % nrb) * RB, r1 = std::min(I, r0 + RB);
        const unsigned char* slab = store + (size_t)e * slab_bytes;
        if (q4x) {
            const uint8_t* qg = slab + lay.w[0];
            const uint8_t* qu = slab + lay.w[1];
            const uint16_t* sg = reinterpret_cast<const uint16_t*>(slab + lay.s[0]);
            const uint16_t* su = reinterpret_cast<const uint16_t*>(slab + lay.s[1]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const uint16_t* xr[4];
                const float* bs[4];
                for (int i = 0; i < nt; ++i) {
                    const int t = order[c0 + i] / k;
                    xr[i] = &xp[(size_t)t * H];
                    bs[i] = &xbs[(size_t)t * (H / 32)];
                }
                const RowPrefetch pq_g(qg, H / 2, I), pq_u(qu, H / 2, I), ps_g(sg, H / 16, I), ps_u(su, H / 16, I);
                for (int r = r0; r < r1; ++r) {
                    pq_g(r), pq_u(r), ps_g(r), ps_u(r);
                    float g[4], u[4];
                    dot_q4x_rows(nt, qg + (size_t)r * (H / 2), sg + (size_t)r * (H / 32), xr, bs, H, g);
                    dot_q4x_rows(nt, qu + (size_t)r * (H / 2), su + (size_t)r * (H / 32), xr, bs, H, u);
                    for (int i = 0; i < nt; ++i)
                        hf[(size_t)order[c0 + i] * I + r] = bf16f(f2bf(g[i] / (1.0f + expf(-g[i])) * u[i]));
                }
            }
            return;
        }
        if (i8_fast) {
            const int8_t* wg = reinterpret_cast<const int8_t*>(slab + lay.w[0]);
            const int8_t* wu = reinterpret_cast<const int8_t*>(slab + lay.w[1]);
            const float* sg = reinterpret_cast<const float*>(slab + lay.s[0]);
            const float* su = reinterpret_cast<const float*>(slab + lay.s[1]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const void* xr[4];
                for (int i = 0; i < nt; ++i) {
                    const size_t o = (size_t)(order[c0 + i] / k) * H;
                    xr[i] = i8_vnni ? (const void*)(reinterpret_cast<const uint8_t*>(xw) + o) : (const void*)&xw[o];
                }
                const RowPrefetch p_g(wg, H, I), p_u(wu, H, I);
                for (int r = r0; r < r1; ++r) {
                    p_g(r), p_u(r);
                    int32_t dg[4], du[4];
                    dot_i8_rows(i8_vnni, nt, wg + (size_t)r * H, xr, H, dg);
                    dot_i8_rows(i8_vnni, nt, wu + (size_t)r * H, xr, H, du);
                    for (int i = 0; i < nt; ++i) {
                        const int p = order[c0 + i], t = p / k;
                        const float g = ((float)dg[i] * xs[t]) * sg[r];
                        const float u = ((float)du[i] * xs[t]) * su[r];
                        hf[(size_t)p * I + r] = (float)(((double)g / (1.0 + exp(-(double)g))) * (double)u);
                    }
                }
            }
            return;
        }
        if (bf16_fast) {
            const uint16_t* wg = reinterpret_cast<const uint16_t*>(slab + lay.w[0]);
            const uint16_t* wu = reinterpret_cast<const uint16_t*>(slab + lay.w[1]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const uint16_t* xr[4];
                for (int i = 0; i < nt; ++i) xr[i] = xb + (size_t)(order[c0 + i] / k) * H;
                const RowPrefetch p_g(wg, (size_t)H * 2, I), p_u(wu, (size_t)H * 2, I);
                for (int r = r0; r < r1; ++r) {
                    p_g(r), p_u(r);
                    float g[4], u[4];
                    dot_bf16x_rows(nt, wg + (size_t)r * H, xr, H, g);
                    dot_bf16x_rows(nt, wu + (size_t)r * H, xr, H, u);
                    for (int i = 0; i < nt; ++i)
                        hf[(size_t)order[c0 + i] * I + r] = bf16f(f2bf(g[i] / (1.0f + expf(-g[i])) * u[i]));
                }
            }
            return;
        }
        for (int r = r0; r < r1; ++r) {
            for (int q = cnt[e]; q < cnt[e + 1]; ++q) {
                const int p = order[q], t = p / k;
                float g, u;
                switch (w_type) {
                    case MOE_W_F32: {
                        const float* wg = reinterpret_cast<const float*>(slab + lay.w[0]) + (size_t)r * H;
                        const float* wu = reinterpret_cast<const float*>(slab + lay.w[1]) + (size_t)r * H;
                        g = dot_f32(wg, xfp + (size_t)t * H, H);
                        u = dot_f32(wu, xfp + (size_t)t * H, H);
                    } break;
                    case MOE_W_BF16: {
                        const uint16_t* wg = reinterpret_cast<const uint16_t*>(slab + lay.w[0]) + (size_t)r * H;
                        const uint16_t* wu = reinterpret_cast<const uint16_t*>(slab + lay.w[1]) + (size_t)r * H;
                        const uint16_t* xr = xb + (size_t)t * H;
                        g = dot_bf16_plain(wg, xr, H);
                        u = dot_bf16_plain(wu, xr, H);
                    } break;
                    case MOE_W_W8A8: {
                        const int8_t* wg = reinterpret_cast<const int8_t*>(slab + lay.w[0]) + (size_t)r * H;
                        const int8_t* wu = reinterpret_cast<const int8_t*>(slab + lay.w[1]) + (size_t)r * H;
                        const float sg = reinterpret_cast<const float*>(slab + lay.s[0])[r];
                        const float su = reinterpret_cast<const float*>(slab + lay.s[1])[r];
                        const int8_t* xr = &xq[(size_t)t * H];
                        g = ((float)dot_i8(wg, xr, H) * xs[t]) * sg;
                        u = ((float)dot_i8(wu, xr, H) * xs[t]) * su;
                    } break;
                    default: {
                        const uint8_t* qg = slab + lay.w[0] + (size_t)r * (H / 2);
                        const uint8_t* qu = slab + lay.w[1] + (size_t)r * (H / 2);
                        const uint16_t* sg = reinterpret_cast<const uint16_t*>(slab + lay.s[0]) + (size_t)r * (H / 32);
                        const uint16_t* su = reinterpret_cast<const uint16_t*>(slab + lay.s[1]) + (size_t)r * (H / 32);
                        if (q4_fast) {
                            const float* bs = &xbs[(size_t)t * (H / 32)];
                            g = dot_q4_avx512(qg, sg, xb + (size_t)t * H, bs, H);
                            u = dot_q4_avx512(qu, su, xb + (size_t)t * H, bs, H);
                        } else {
                            g = dot_q4(qg, sg, xfp + (size_t)t * H, H);
                            u = dot_q4(qu, su, xfp + (size_t)t * H, H);
                        }
                    } break;
                }
                float h;
                if (w_type == MOE_W_W8A8) h = (float)(((double)g / (1.0 + exp(-(double)g))) * (double)u);
                else h = g / (1.0f + expf(-g)) * u;
                if (w_type == MOE_W_BF16 || w_type == MOE_W_Q4B32) h = bf16f(f2bf(h));
                hf[(size_t)p * I + r] = h;
            }
        }
    });

    // per-pick forms of h, one pick per work item: int8 with its scale and
    // widened (W8A8), bf16 bits (bf16, 4-bit), and for 4-bit the block sums
    // and the grouped order
    const std::function<void(int)> prep_pick = [&](int q) {
        const int p = order[q];
        const float* hr = &hf[(size_t)p * I];
        if (w_type == MOE_W_W8A8) {
            hs[p] = quant_row(hr, I, &hq[(size_t)p * I]);
            if (i8_vnni) {
                uint8_t* hu = reinterpret_cast<uint8_t*>(hw) + (size_t)p * I;
                for (int i = 0; i < I; ++i) hu[i] = (uint8_t)(hq[(size_t)p * I + i] + 128);
            } else if (i8_fast) {
                for (int i = 0; i < I; ++i) hw[(size_t)p * I + i] = hq[(size_t)p * I + i];
            }
        }
        if (need_hb)
            for (int i = 0; i < I; ++i) hb[(size_t)p * I + i] = f2bf(hr[i]);
        if (q4_fast) block_sums(&hb[(size_t)p * I], I, &hbs[(size_t)p * (I / 32)]);
        if (q4x) q4x_order(&hb[(size_t)p * I], I, &hp[(size_t)p * I]);
    };
    if (w_type != MOE_W_F32) {
        const int nq = (int)order.size();
        if (nq >= 8) parallel(n_threads, nq, prep_pick);
        else
            for (int q = 0; q < nq; ++q) prep_pick(q);
    }

    // phase 2: down rows -> part[p][m] = w * o
    const int RD = 64;
    const int nrd = (H + RD - 1) / RD;
    parallel(n_threads, NE * nrd, [&](int item) {
        const int e = experts[item / nrd], m0 = (item % nrd) * RD, m1 = std::min(H, m0 + RD);
        const unsigned char* slab = store + (size_t)e * slab_bytes;
        if (q4x) {
            const uint8_t* qd = slab + lay.w[2];
            const uint16_t* sd = reinterpret_cast<const uint16_t*>(slab + lay.s[2]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const uint16_t* hr[4];
                const float* bs[4];
                for (int i = 0; i < nt; ++i) {
                    hr[i] = &hp[(size_t)order[c0 + i] * I];
                    bs[i] = &hbs[(size_t)order[c0 + i] * (I / 32)];
                }
                const RowPrefetch pq(qd, I / 2, H), ps(sd, I / 16, H);
                for (int m = m0; m < m1; ++m) {
                    pq(m), ps(m);
                    float o[4];
                    dot_q4x_rows(nt, qd + (size_t)m * (I / 2), sd + (size_t)m * (I / 32), hr, bs, I, o);
                    for (int i = 0; i < nt; ++i) {
                        const int p = order[c0 + i];
                        part[(size_t)p * H + m] = w_h[p] * o[i];
                    }
                }
            }
            return;
        }
        if (i8_fast) {
            const int8_t* wd = reinterpret_cast<const int8_t*>(slab + lay.w[2]);
            const float* sd = reinterpret_cast<const float*>(slab + lay.s[2]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const void* hr[4];
                for (int i = 0; i < nt; ++i) {
                    const size_t o = (size_t)order[c0 + i] * I;
                    hr[i] = i8_vnni ? (const void*)(reinterpret_cast<const uint8_t*>(hw) + o) : (const void*)&hw[o];
                }
                const RowPrefetch pw(wd, I, H);
                for (int m = m0; m < m1; ++m) {
                    pw(m);
                    int32_t d[4];
                    dot_i8_rows(i8_vnni, nt, wd + (size_t)m * I, hr, I, d);
                    for (int i = 0; i < nt; ++i) {
                        const int p = order[c0 + i];
                        part[(size_t)p * H + m] = w_h[p] * (((float)d[i] * hs[p]) * sd[m]);
                    }
                }
            }
            return;
        }
        if (bf16_fast) {
            const uint16_t* wd = reinterpret_cast<const uint16_t*>(slab + lay.w[2]);
            for (int c0 = cnt[e]; c0 < cnt[e + 1]; c0 += 4) {
                const int nt = std::min(4, cnt[e + 1] - c0);
                const uint16_t* hr[4];
                for (int i = 0; i < nt; ++i) hr[i] = &hb[(size_t)order[c0 + i] * I];
                const RowPrefetch pw(wd, (size_t)I * 2, H);
                for (int m = m0; m < m1; ++m) {
                    pw(m);
                    float o[4];
                    dot_bf16x_rows(nt, wd + (size_t)m * I, hr, I, o);
                    for (int i = 0; i < nt; ++i) {
                        const int p = order[c0 + i];
                        part[(size_t)p * H + m] = w_h[p] * o[i];
                    }
                }
            }
            return;
        }
        for (int m = m0; m < m1; ++m) {
            for (int q = cnt[e]; q < cnt[e + 1]; ++q) {
                const int p = order[q];
                float o;
                switch (w_type) {
                    case MOE_W_F32:
                        o = dot_f32(reinterpret_cast<const float*>(slab + lay.w[2]) + (size_t)m * I, &hf[(size_t)p * I], I);
                        break;
                    case MOE_W_BF16: {
                        const uint16_t* wd = reinterpret_cast<const uint16_t*>(slab + lay.w[2]) + (size_t)m * I;
                        float a = 0.0f;
                        for (int i = 0; i < I; ++i) a += bf16f(wd[i]) * hf[(size_t)p * I + i];
                        o = a;
                    } break;
                    case MOE_W_W8A8: {
                        const int8_t* wd = reinterpret_cast<const int8_t*>(slab + lay.w[2]) + (size_t)m * I;
                        const float sd = reinterpret_cast<const float*>(slab + lay.s[2])[m];
                        const int8_t* hr = &hq[(size_t)p * I];
                        o = ((float)dot_i8(wd, hr, I) * hs[p]) * sd;
                    } break;
                    default: {
                        const uint8_t* qd = slab + lay.w[2] + (size_t)m * (I / 2);
                        const uint16_t* sd = reinterpret_cast<const uint16_t*>(slab + lay.s[2]) + (size_t)m * (I / 32);
                        o = q4_fast ? dot_q4_avx512(qd, sd, &hb[(size_t)p * I], &hbs[(size_t)p * (I / 32)], I)
                                    : dot_q4(qd, sd, &hf[(size_t)p * I], I);
                    } break;
                }
                part[(size_t)p * H + m] = w_h[p] * o;
            }
        }
    });

    // phase 3: y[t] = sum over non-resident picks, j ascending
    parallel(n_threads, T, [&](int t) {
        float* yr = y_h + (size_t)t * H;
        for (int m = 0; m < H; ++m) yr[m] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            if (slot_ids_h[p] >= 0 || ids_h[p] < 0 || ids_h[p] >= E) continue;
            const float* pr = &part[(size_t)p * H];
            for (int m = 0; m < H; ++m) yr[m] += pr[m];
        }
    });
    return moe_ok();
}

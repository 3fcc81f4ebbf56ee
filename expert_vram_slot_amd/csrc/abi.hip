// Error state, version, slab layout and pinned host memory of the C ABI.
#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "common.hpp"

static thread_local char g_err[512] = "";

int moe_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int moe_ok() {
    g_err[0] = 0;
    return MOE_OK;
}

int moe_check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return moe_fail(MOE_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return moe_ok();
}

int moe_layout(int w_type, int H, int I, moe_slab_layout_t* out) {
    if (!out) return moe_fail(MOE_E_ARG, "moe_slab_layout: out is NULL");
    if (H <= 0 || I <= 0) return moe_fail(MOE_E_ARG, "moe_slab_layout: H=%d I=%d must be positive", H, I);
    const int64_t n = (int64_t)H * I;
    for (int p = 0; p < 3; ++p) out->s[p] = -1;
    switch (w_type) {
        case MOE_W_F32:
        case MOE_W_BF16: {
            if (H % 16 || I % 16)
                return moe_fail(MOE_E_ALIGN, "moe_slab_layout: H=%d and I=%d must be multiples of 16", H, I);
            const int64_t es = w_type == MOE_W_F32 ? 4 : 2;
            for (int p = 0; p < 3; ++p) out->w[p] = p * n * es;
            out->total = 3 * n * es;
        } break;
        case MOE_W_W8A8: {
            if (H % 16 || I % 16)
                return moe_fail(MOE_E_ALIGN, "moe_slab_layout: H=%d and I=%d must be multiples of 16", H, I);
            for (int p = 0; p < 3; ++p) out->w[p] = p * n;
            out->s[0] = 3 * n;
            out->s[1] = 3 * n + 4 * (int64_t)I;
            out->s[2] = 3 * n + 8 * (int64_t)I;
            out->total = 3 * n + 4 * (2 * (int64_t)I + H);
        } break;
        case MOE_W_Q4B32: {
            if (H % 32 || I % 32)
                return moe_fail(MOE_E_ALIGN, "moe_slab_layout: 4-bit blocks need H=%d and I=%d multiples of 32", H, I);
            // both planes must start on 16 bytes: rows*cols/16 (the scale plane) must be a multiple of 16
            if (n % 256)
                return moe_fail(MOE_E_ALIGN, "moe_slab_layout: H*I=%lld must be a multiple of 256", (long long)n);
            const int64_t nib = n / 2, sc = n / 16;
            for (int p = 0; p < 3; ++p) {
                out->w[p] = p * (nib + sc);
                out->s[p] = out->w[p] + nib;
            }
            out->total = 3 * (nib + sc);
        } break;
        default:
            return moe_fail(MOE_E_DTYPE, "moe_slab_layout: unknown weight format %d", w_type);
    }
    return moe_ok();
}

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

int moe_slab_layout(int w_type, int H, int I, moe_slab_layout_t* out) { return moe_layout(w_type, H, I, out); }

void* moe_host_alloc(size_t bytes) {
    void* p = nullptr;
    if (bytes == 0) {
        moe_fail(MOE_E_ARG, "moe_host_alloc: zero bytes");
        return nullptr;
    }
    hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) {
        moe_fail(MOE_E_NOMEM, "moe_host_alloc: hipHostMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
        return nullptr;
    }
    moe_ok();
    return p;
}

int moe_host_free(void* p) {
    if (!p) return moe_ok();
    hipError_t e = hipHostFree(p);
    if (e != hipSuccess) return moe_fail(MOE_E_HIP, "moe_host_free: %s", hipGetErrorString(e));
    return moe_ok();
}

}  // extern "C"

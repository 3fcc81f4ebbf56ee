// Residual join between stacked MoE layers: x_next = bf16(x + y).
//
// "Nudge, don't cut" (oois.ee/pgo-sgb), "Experts that don't fit": the routed
// layers sit one after another in a 48-layer model; each layer's output is
// added to the stream it read.  The stream is kept in bf16 (the activations'
// storage format), the add is done in fp32 and rounded to nearest even.
#include "common.hpp"

namespace {

__global__ void __launch_bounds__(256) k_residual_bf16(const uint16_t* __restrict__ x, const float* __restrict__ y,
                                                       uint16_t* __restrict__ out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = moe::f32_to_bf16(moe::bf16_to_f32(x[i]) + y[i]);
}

__global__ void __launch_bounds__(256) k_residual_f32(const float* __restrict__ x, const float* __restrict__ y,
                                                      float* __restrict__ out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = x[i] + y[i];
}

}  // namespace

extern "C" int moe_residual(const void* x, int x_dtype, const float* y, void* x_out, int T, int H,
                            hipStream_t stream) {
    MOE_REQUIRE(x && y && x_out && T >= 0 && H >= 1, MOE_E_ARG, "moe_residual: bad arguments");
    MOE_REQUIRE(x_dtype == MOE_X_F32 || x_dtype == MOE_X_BF16, MOE_E_DTYPE, "moe_residual: activation format %d",
                x_dtype);
    const int64_t n = (int64_t)T * H;
    if (n == 0) return moe_ok();
    const dim3 grid((unsigned)((n + 255) / 256));
    if (x_dtype == MOE_X_BF16)
        hipLaunchKernelGGL(k_residual_bf16, grid, dim3(256), 0, stream, reinterpret_cast<const uint16_t*>(x), y,
                           reinterpret_cast<uint16_t*>(x_out), n);
    else
        hipLaunchKernelGGL(k_residual_f32, grid, dim3(256), 0, stream, reinterpret_cast<const float*>(x), y,
                           reinterpret_cast<float*>(x_out), n);
    return moe_check_launch("moe_residual");
}

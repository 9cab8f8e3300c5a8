// moe_swiglu_backward: gradient of h = silu(g) * u with respect to the saved gate and up
// pre-activations, for every row of the grouped MLP at once.
//
// [Blog] Figure 3 paragraph: each expert is a SwiGLU MLP (gate and up projections, then
// the down projection); the backward of the expert stack runs the SwiGLU derivative between
// the two data-gradient GEMMs. With s = sigmoid(g):
//   dg = dh * u * s * (1 + g * (1 - s))      (the derivative of silu(g) = g * s)
//   du = dh * g * s
// Elementwise and bandwidth-bound: each thread handles 8 consecutive columns (16-byte
// loads of dh, g and u, 16-byte stores of dg and du), math in fp32, one rounding per output.
#include "moe_internal.h"
#include "swiglu_math.h"

namespace moe {
namespace {

template <int ESIZE>
__device__ __forceinline__ void ld8(const char* p, float (&v)[8]) {
    if (ESIZE == 2) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));   // read once
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(q[i] << 16);
            v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
        }
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(p);
        const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    }
}

template <int ESIZE>
__device__ __forceinline__ void st8(char* p, const float (&v)[8]) {
    if (ESIZE == 2) {
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));                      // written once
    } else {
        u32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = __float_as_uint(v[i]);
            b[i] = __float_as_uint(v[4 + i]);
        }
        *reinterpret_cast<u32x4*>(p) = a;
        *reinterpret_cast<u32x4*>(p + 16) = b;
    }
}

template <int ESIZE>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const char* __restrict__ dh, int64_t ld_dh,
                                                         const char* __restrict__ gu, int64_t ld_gu,
                                                         char* __restrict__ dgu, int64_t ld_dgu, int64_t rows,
                                                         int f) {
    const int per_row = f / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * per_row) return;
    const int64_t r = idx / per_row;
    const int c = (int)(idx % per_row) * 8;
    float h[8], g[8], u[8], dg[8], du[8];
    ld8<ESIZE>(dh + (r * ld_dh + c) * ESIZE, h);
    ld8<ESIZE>(gu + (r * ld_gu + c) * ESIZE, g);
    ld8<ESIZE>(gu + (r * ld_gu + f + c) * ESIZE, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) swiglu_grad(h[i], g[i], u[i], dg[i], du[i]);
    st8<ESIZE>(dgu + (r * ld_dgu + c) * ESIZE, dg);
    st8<ESIZE>(dgu + (r * ld_dgu + f + c) * ESIZE, du);
}

}  // namespace
}  // namespace moe

extern "C" moe_status_t moe_swiglu_backward(const void* dh, int64_t ld_dh, const void* gu, int64_t ld_gu,
                                            int32_t dtype, int64_t rows, int64_t f, void* dgu, int64_t ld_dgu,
                                            void* stream) {
    if (rows < 0 || f <= 0 || f % 8 != 0 || f > INT32_MAX / 4) return MOE_EINVAL;
    if (ld_dh < f || ld_gu < 2 * f || ld_dgu < 2 * f || ld_dh % 8 || ld_gu % 8 || ld_dgu % 8) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (rows == 0) return MOE_OK;
    if (!dh || !gu || !dgu || !moe_aligned16(dh) || !moe_aligned16(gu) || !moe_aligned16(dgu)) return MOE_EINVAL;
    const int64_t n = rows * (f / 8);
    const dim3 grid((unsigned)moe::cdiv<int64_t>(n, 256));
    hipStream_t s = (hipStream_t)stream;
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(moe::swiglu_bwd_kernel<2>, grid, dim3(256), 0, s, (const char*)dh, ld_dh,
                           (const char*)gu, ld_gu, (char*)dgu, ld_dgu, rows, (int)f);
    else
        hipLaunchKernelGGL(moe::swiglu_bwd_kernel<4>, grid, dim3(256), 0, s, (const char*)dh, ld_dh,
                           (const char*)gu, ld_gu, (char*)dgu, ld_dgu, rows, (int)f);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

// moe_combine: return every expert output row to its token and sum them with the routing
// weights (plus the always-on shared expert), in a fixed order with fp32 accumulation.
// With no weights it is the transpose of the permutation (dx[t] = sum_j dX_perm[row_of[t,j]]).
// moe_combine_backward: the transpose of the weighted combine (dY rows and the routing
// weights' gradient).
//
// [Blog] "Optimisation 2": combine brings each processed token back to its original
// position and accumulates the experts' results. Written as a gather-reduce per token
// rather than a scatter-add: every output element is produced by exactly one lane, so the
// result is deterministic and needs no atomics or zero-initialised output.
#include <algorithm>

#include "moe_internal.h"
#include "round_math.h"

namespace moe {
namespace {

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1   // expert rows are read once: non-temporal loads (measured 230 -> 203 us at DeepSeek-V3 size)
#endif

constexpr int kCombThreads = 256;

__device__ __forceinline__ u32x4 ld_row16(const char* p) {
    if constexpr (MOE_COMBINE_NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}
constexpr int kCombMaxThreads = 512;   // forward combine: block sized to the row (see comb_threads)

template <int ESIZE>
__device__ __forceinline__ void load8(const char* p, float (&v)[8]) {
    if (ESIZE == 2) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(p);
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
__device__ __forceinline__ void store8(char* p, const float (&v)[8]) {
    if (ESIZE == 2) {
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4*>(p) = q;
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
__device__ __forceinline__ void cvt8(const u32x4& a, const u32x4& b, float (&v)[8]) {
    if (ESIZE == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(a[i] << 16);
            v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    }
}

// One workgroup per token; each thread owns 8 consecutive columns at a time. KK > 0 is the
// number of routed rows per token known at compile time: then the KK row loads (and the
// shared expert's) are all issued before the first one is used, so a lane keeps KK+1 loads
// in flight instead of one. The fp32 sum runs in the same order either way (slot 0 .. k-1,
// then the shared row), so every KK gives the same bits.
template <int ESIZE, int KK>
__global__ __launch_bounds__(kCombMaxThreads) void combine_kernel(const char* __restrict__ y,
                                                               const float* __restrict__ topk_w,
                                                               const int32_t* __restrict__ row_of,
                                                               const char* __restrict__ y_shared, int T, int d,
                                                               int k, char* __restrict__ out) {
    const int t = blockIdx.x;
    __shared__ int rows[16];
    __shared__ float wts[16];
    const int TK = T * k;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = min(max(row_of[(int64_t)t * k + threadIdx.x], 0), TK - 1);
        wts[threadIdx.x] = topk_w ? topk_w[(int64_t)t * k + threadIdx.x] : 1.f;   // NULL: plain sum
    }
    __syncthreads();
    const int ngroups = d / 8;
    const int64_t rowbytes = (int64_t)d * ESIZE;
    if constexpr (KK > 0) {
        for (int c = threadIdx.x; c < ngroups; c += blockDim.x) {
            const int64_t col = (int64_t)c * 8 * ESIZE;
            u32x4 ra[KK], rb[KK], sa = {}, sb = {};
#pragma unroll
            for (int j = 0; j < KK; ++j) {
                const char* src = y + rows[j] * rowbytes + col;
                ra[j] = ld_row16(src);
                if (ESIZE == 4) rb[j] = ld_row16(src + 16);
            }
            if (y_shared != nullptr) {
                const char* src = y_shared + t * rowbytes + col;
                sa = ld_row16(src);
                if (ESIZE == 4) sb = ld_row16(src + 16);
            }
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KK; ++j) {
                float v[8];
                cvt8<ESIZE>(ra[j], rb[j], v);
                const float w = wts[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
            }
            if (y_shared != nullptr) {
                float v[8];
                cvt8<ESIZE>(sa, sb, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += v[i];
            }
            store8<ESIZE>(out + t * rowbytes + col, acc);
        }
        return;
    }
    for (int c = threadIdx.x; c < ngroups; c += blockDim.x) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            float v[8];
            load8<ESIZE>(y + rows[j] * rowbytes + c * 8 * ESIZE, v);
            const float w = wts[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
        }
        if (y_shared != nullptr) {
            float v[8];
            load8<ESIZE>(y_shared + t * rowbytes + c * 8 * ESIZE, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        store8<ESIZE>(out + t * rowbytes + c * 8 * ESIZE, acc);
    }
}


// Transpose of the combine, one workgroup per token:
//   dy[row_of[t,j]] = w[t,j] * d_out[t]       (every routed row is written exactly once)
//   dy_shared[t]    = d_out[t]                (the shared expert's output gradient)
//   dw[t,j]         = <d_out[t], y[row_of[t,j]]>   (fp32, fixed reduction order)
template <int ESIZE>
__global__ __launch_bounds__(kCombThreads) void combine_bwd_kernel(const char* __restrict__ d_out,
                                                                   const float* __restrict__ topk_w,
                                                                   const int32_t* __restrict__ row_of,
                                                                   const char* __restrict__ y, int T, int d, int k,
                                                                   char* __restrict__ dy, char* __restrict__ dy_shared,
                                                                   float* __restrict__ dw) {
    const int t = blockIdx.x;
    __shared__ int rows[16];
    __shared__ float wts[16];
    __shared__ float red[kCombThreads / kWave][16];
    const int TK = T * k;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = min(max(row_of[(int64_t)t * k + threadIdx.x], 0), TK - 1);
        wts[threadIdx.x] = topk_w[(int64_t)t * k + threadIdx.x];
    }
    __syncthreads();
    const int ngroups = d / 8;
    const int64_t rowbytes = (int64_t)d * ESIZE;
    float part[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) part[j] = 0.f;
    for (int c = threadIdx.x; c < ngroups; c += kCombThreads) {
        float g[8];
        load8<ESIZE>(d_out + t * rowbytes + c * 8 * ESIZE, g);
        if (dy_shared != nullptr) store8<ESIZE>(dy_shared + t * rowbytes + c * 8 * ESIZE, g);
        // the slots in batches of 8: the batch's expert rows of y are all loaded (slot index
        // clamped, so every load is valid and issued together) before any is used
        for (int j0 = 0; j0 < k; j0 += 8) {
            float v[8][8];
            if (dw != nullptr) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    load8<ESIZE>(y + rows[min(j0 + u, k - 1)] * rowbytes + c * 8 * ESIZE, v[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j >= k) break;
                float o[8];
                const float w = wts[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = ESIZE == 2 ? mul_round_odd(w, g[i]) : w * g[i];
                if (dy != nullptr) store8<ESIZE>(dy + rows[j] * rowbytes + c * 8 * ESIZE, o);
                if (dw != nullptr) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = fmaf(g[i], v[u][i], acc);
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        if (q == j) part[q] += acc;
                }
            }
        }
    }
    if (dw == nullptr) return;
    // fixed-order reduction: wave butterfly, then the 4 waves in order
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j >= k) break;
        float v = part[j];
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
        if (lane == 0) red[wave][j] = v;
    }
    __syncthreads();
    if (threadIdx.x < k) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kCombThreads / kWave; ++w) v += red[w][threadIdx.x];
        dw[(int64_t)t * k + threadIdx.x] = v;
    }
}

// Threads per token: whole waves, as few passes over the row's 8-column groups as 512
// threads allow, split evenly (d = 7168: 896 groups -> 448 threads x 2 passes, where 256
// threads would leave half of them idle in the last pass).
inline int comb_threads(int64_t d) {
    const int64_t groups = d / 8;
    const int64_t passes = cdiv<int64_t>(groups, kCombMaxThreads);
    return (int)std::min<int64_t>(kCombMaxThreads, std::max<int64_t>(kWave, kWave * cdiv<int64_t>(cdiv<int64_t>(groups, passes), kWave)));
}

template <int ESIZE>
void launch_combine(int k, const char* y, const float* topk_w, const int32_t* row_of, const char* y_shared,
                    int64_t T, int64_t d, char* out, hipStream_t s) {
    const dim3 grid((unsigned)T), block((unsigned)comb_threads(d));
    switch (k) {
        case 1: hipLaunchKernelGGL((combine_kernel<ESIZE, 1>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
        case 2: hipLaunchKernelGGL((combine_kernel<ESIZE, 2>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
        case 4: hipLaunchKernelGGL((combine_kernel<ESIZE, 4>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
        case 6: hipLaunchKernelGGL((combine_kernel<ESIZE, 6>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
        case 8: hipLaunchKernelGGL((combine_kernel<ESIZE, 8>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
        default: hipLaunchKernelGGL((combine_kernel<ESIZE, 0>), grid, block, 0, s, y, topk_w, row_of, y_shared, (int)T, (int)d, k, out); break;
    }
}

}  // namespace
}  // namespace moe

extern "C" moe_status_t moe_combine_backward(const void* d_out, int32_t dtype, const float* topk_w,
                                             const int32_t* row_of, const void* y, int64_t T, int64_t d, int32_t k,
                                             void* dy, void* dy_shared, float* dw, void* stream) {
    if (T < 0 || d <= 0 || d % 8 != 0 || k < 1 || k > 16) return MOE_EINVAL;
    if (T * (int64_t)k > INT32_MAX || d > INT32_MAX / 16) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!d_out || !topk_w || !row_of || (dw && !y)) return MOE_EINVAL;
    if (!moe_aligned16(d_out) || (dy && !moe_aligned16(dy)) || (dy_shared && !moe_aligned16(dy_shared)) ||
        (dw && !moe_aligned16(y)))
        return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(moe::combine_bwd_kernel<2>, dim3((unsigned)T), dim3(moe::kCombThreads), 0, s,
                           (const char*)d_out, topk_w, row_of, (const char*)y, (int)T, (int)d, k, (char*)dy,
                           (char*)dy_shared, dw);
    else
        hipLaunchKernelGGL(moe::combine_bwd_kernel<4>, dim3((unsigned)T), dim3(moe::kCombThreads), 0, s,
                           (const char*)d_out, topk_w, row_of, (const char*)y, (int)T, (int)d, k, (char*)dy,
                           (char*)dy_shared, dw);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" moe_status_t moe_combine(const void* y, int32_t dtype, const float* topk_w, const int32_t* row_of,
                                    const void* y_shared, int64_t T, int64_t d, int32_t k, void* out,
                                    void* stream) {
    if (T < 0 || d <= 0 || d % 8 != 0 || k < 1 || k > 16) return MOE_EINVAL;
    if (T * (int64_t)k > INT32_MAX || d > INT32_MAX / 16) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!y || !row_of || !out) return MOE_EINVAL;
    if (!moe_aligned16(y) || !moe_aligned16(out) || (y_shared && !moe_aligned16(y_shared))) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == MOE_BF16) moe::launch_combine<2>(k, (const char*)y, topk_w, row_of, (const char*)y_shared, T, d, (char*)out, s);
    else moe::launch_combine<4>(k, (const char*)y, topk_w, row_of, (const char*)y_shared, T, d, (char*)out, s);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

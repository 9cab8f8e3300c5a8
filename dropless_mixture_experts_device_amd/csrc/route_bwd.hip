// moe_route_backward: the router's backward. Given the gradient of the loss with respect to
// the normalised top-k routing weights (the combine's backward produces it), it forms the
// gradient of the selected keys and from it the gradients of the router weights, the expert
// bias and the router's share of the input gradient.
//
// [Blog] opening section: a learnable router picks each token's top-K experts; the router is
// trained with the rest of the layer. The selection is piecewise constant in the keys, so only
// the selected experts' keys receive gradient:
//   softmax: w = softmax over the selected keys,  dk_j = w_j (g_j - sum_i w_i g_i)
//   sigmoid: w_j = s_j / S, s_j = sigmoid(k_j),    dk_j = (g_j - sum_i w_i g_i) / S * s_j (1 - s_j)
// and with the keys = x W_r^T + b:
//   dW_r[e] = sum over tokens t that selected e of dk[t,e] x[t]   (fp32; the expert's rows in
//             the permutation's ascending token order, in chunks of 256 rows whose partial
//             sums are then added in chunk order)
//   d_bias[e] = sum of the same dk[t,e]                             (fp32, fixed-order tree)
//   dx[t]   = sum_j dk[t,j] W_r[S_tj]                                (fp32 sum in slot order,
//             one rounding to the input dtype)
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRbThreads = 256;
constexpr int kRbCols = kRbThreads * 8;   // columns of dW_r per workgroup (8 per thread)
constexpr int kRbChunk = 256;             // permuted rows per weight-gradient partial sum

__host__ __device__ inline size_t rb_align(size_t v) { return (v + 255) & ~size_t(255); }

// One thread per token: the k selected keys' gradient, written per slot and per permuted row.
__global__ __launch_bounds__(kRbThreads) void route_bwd_keys_kernel(const float* __restrict__ keys,
                                                                    const int32_t* __restrict__ topk_idx,
                                                                    const float* __restrict__ d_w,
                                                                    const int32_t* __restrict__ row_of, int T,
                                                                    int E, int k, int score, int TK,
                                                                    float* __restrict__ dk_sel,
                                                                    float* __restrict__ dk_perm) {
    const int t = blockIdx.x * kRbThreads + threadIdx.x;
    if (t >= T) return;
    float kk[16], g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < k) {
            const int e = min(max(topk_idx[(int64_t)t * k + j], 0), E - 1);
            kk[j] = keys[(int64_t)t * E + e];
            g[j] = d_w[(int64_t)t * k + j];
        } else {
            kk[j] = 0.f;
            g[j] = 0.f;
        }
    }
    // the weights as the forward forms them, then the common term sum_i w_i g_i. For the
    // sigmoid, 1 - s_j is taken as sigmoid(-key_j) rather than by subtraction, which would
    // lose the low bits of s_j (1 - s_j) once s_j is close to one.
    float z[16], zc[16], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        z[j] = 0.f;
        zc[j] = 0.f;
        if (j < k) {
            if (score == MOE_SOFTMAX) {
                z[j] = expf(kk[j] - kk[0]);
            } else {
                z[j] = 1.0f / (1.0f + expf(-kk[j]));
                zc[j] = 1.0f / (1.0f + expf(kk[j]));
            }
            sum += z[j];
        }
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (j < k) dot += (z[j] / sum) * g[j];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < k) {
            const float dk = (score == MOE_SOFTMAX) ? (z[j] / sum) * (g[j] - dot)
                                                    : (g[j] - dot) / sum * z[j] * zc[j];
            dk_sel[(int64_t)t * k + j] = dk;
            const int r = min(max(row_of[(int64_t)t * k + j], 0), TK - 1);
            dk_perm[r] = dk;
        }
    }
}

template <int ESIZE>
__device__ __forceinline__ void ld8f(const char* p, float (&v)[8]) {
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

// dx[t] = sum_j dk[t,j] W_r[S_tj]: one workgroup per token, 8 columns per thread per pass.
template <int ESIZE>
__global__ __launch_bounds__(kRbThreads) void route_bwd_dx_kernel(const char* __restrict__ w_router,
                                                                  const int32_t* __restrict__ topk_idx,
                                                                  const float* __restrict__ dk_sel, int d, int E,
                                                                  int k, int accumulate, char* __restrict__ dx,
                                                                  const char* __restrict__ dxp,
                                                                  const char* __restrict__ dxp_shared,
                                                                  const int32_t* __restrict__ row_of, int TK) {
    const int t = blockIdx.x;
    __shared__ int rows[16];
    __shared__ int prow[16];
    __shared__ float coef[16];
    if (threadIdx.x < k) {
        rows[threadIdx.x] = min(max(topk_idx[(int64_t)t * k + threadIdx.x], 0), E - 1);
        coef[threadIdx.x] = dk_sel[(int64_t)t * k + threadIdx.x];
        if (dxp != nullptr) prow[threadIdx.x] = min(max(row_of[(int64_t)t * k + threadIdx.x], 0), TK - 1);
    }
    __syncthreads();
    const int64_t rowbytes = (int64_t)d * ESIZE;
    for (int c = threadIdx.x; c < d / 8; c += kRbThreads) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += 8) {   // batches of 8 slots, every row load issued first
            float v[8][8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                ld8f<ESIZE>(w_router + rows[min(j0 + u, k - 1)] * rowbytes + (int64_t)c * 8 * ESIZE, v[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) {   // slots past k repeat a finite row with weight zero
                const float w = j0 + u < k ? coef[min(j0 + u, 15)] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[u][i], acc[i]);
            }
        }
        char* o = dx + t * rowbytes + (int64_t)c * 8 * ESIZE;
        if (dxp != nullptr) {
            // the incoming gradient formed here as the permutation's transpose: the token's
            // permuted rows summed in fp32 in slot order, then its shared row, rounded once to
            // the storage type (exactly what moe_combine without weights stores)
            float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j0 = 0; j0 < k; j0 += 8) {
                float v[8][8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    ld8f<ESIZE>(dxp + prow[min(j0 + u, k - 1)] * rowbytes + (int64_t)c * 8 * ESIZE, v[u]);
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int i = 0; i < 8; ++i) sum[i] = j0 + u < k ? fmaf(1.f, v[u][i], sum[i]) : sum[i];
            }
            if (dxp_shared != nullptr) {
                float v[8];
                ld8f<ESIZE>(dxp_shared + t * rowbytes + (int64_t)c * 8 * ESIZE, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) sum[i] += v[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += ESIZE == 2 ? bf16_to_f32(f32_to_bf16(sum[i])) : sum[i];
        } else if (accumulate) {   // the incoming gradient joins the fp32 sum; still one rounding
            float v[8];
            ld8f<ESIZE>(o, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        if (ESIZE == 2) {
            u32x4 q;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                q[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
            *reinterpret_cast<u32x4*>(o) = q;
        } else {
            u32x4 a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = __float_as_uint(acc[i]);
                b[i] = __float_as_uint(acc[4 + i]);
            }
            *reinterpret_cast<u32x4*>(o) = a;
            *reinterpret_cast<u32x4*>(o + 16) = b;
        }
    }
}

// Each expert's group of permuted rows is cut into chunks of kRbChunk rows, so a hot
// expert's rows spread over many workgroups. chunk_off[e] = number of chunks of experts < e.
__global__ __launch_bounds__(kRbThreads) void route_bwd_chunks_kernel(const int32_t* __restrict__ offsets, int E,
                                                                      int TK, int32_t* __restrict__ chunk_off) {
    __shared__ int c[kRbThreads];
    const int e = threadIdx.x;
    int n = 0;
    if (e < E) {
        const int rb = min(max(offsets[e], 0), TK);
        const int re = min(max(offsets[e + 1], rb), TK);
        n = cdiv(re - rb, kRbChunk);
    }
    c[e] = n;
    __syncthreads();
    for (int h = 1; h < kRbThreads; h <<= 1) {   // inclusive scan
        const int v = e >= h ? c[e - h] : 0;
        __syncthreads();
        c[e] += v;
        __syncthreads();
    }
    if (e == 0) chunk_off[0] = 0;
    if (e < E) chunk_off[e + 1] = c[e];
}

// partial[chunk, cols] = sum over the chunk's rows (ascending) of dk[r] * x[src_token[r], cols];
// rows are taken four at a time. Workgroups past the last chunk exit at once.
template <int ESIZE>
__global__ __launch_bounds__(kRbThreads) void route_bwd_dw_partial_kernel(const char* __restrict__ x,
                                                                          const int32_t* __restrict__ offsets,
                                                                          const int32_t* __restrict__ chunk_off,
                                                                          const int32_t* __restrict__ src_token,
                                                                          const float* __restrict__ dk_perm, int T,
                                                                          int d, int E, int TK,
                                                                          float* __restrict__ partial) {
    const int ch = blockIdx.x;
    if (ch >= chunk_off[E]) return;
    int lo = 0, hi = E - 1;   // the expert whose chunks hold ch: largest e with chunk_off[e] <= ch
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= ch) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int rb = min(max(offsets[e], 0), TK);
    const int re = min(max(offsets[e + 1], rb), TK);
    const int r_begin = min(rb + (ch - chunk_off[e]) * kRbChunk, re);
    const int r_end = min(r_begin + kRbChunk, re);
    const int col = blockIdx.y * kRbCols + threadIdx.x * 8;
    if (col >= d) return;
    const int64_t rowbytes = (int64_t)d * ESIZE;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // four rows per step; loads guarded by the row bound (a batched form with clamped rows
    // and eight loads in flight measured slower here: 134 -> 157 us at the DeepSeek-V3 shape)
    constexpr int U = 4;
    for (int r0 = r_begin; r0 < r_end; r0 += U) {
        float v[U][8], c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u;
            c[u] = 0.f;
            if (r < r_end) {
                const int tok = min(max(src_token[r], 0), T - 1);
                c[u] = dk_perm[r];
                ld8f<ESIZE>(x + tok * rowbytes + (int64_t)col * ESIZE, v[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (r0 + u < r_end)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(c[u], v[u][i], acc[i]);
    }
    float* o = partial + (int64_t)ch * d + col;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// dW_r[e, cols] = expert e's chunk partials summed in chunk order (zero for an empty group);
// d_bias[e] from the workgroups of the first column block (fixed-order tree over the rows).
__global__ __launch_bounds__(kRbThreads) void route_bwd_dw_reduce_kernel(const float* __restrict__ partial,
                                                                         const int32_t* __restrict__ offsets,
                                                                         const int32_t* __restrict__ chunk_off,
                                                                         const float* __restrict__ dk_perm, int d,
                                                                         int TK, int max_chunks,
                                                                         float* __restrict__ dw,
                                                                         float* __restrict__ dbias) {
    const int e = blockIdx.x;
    const int col = blockIdx.y * kRbCols + threadIdx.x * 8;
    if (dw != nullptr && col < d) {
        const int c0 = min(chunk_off[e], max_chunks);
        const int c1 = min(max(chunk_off[e + 1], c0), max_chunks);
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        for (int c = c0; c < c1; ++c) {
            const float* p = partial + (int64_t)c * d + col;
            a += *reinterpret_cast<const f32x4*>(p);
            b += *reinterpret_cast<const f32x4*>(p + 4);
        }
        float* o = dw + (int64_t)e * d + col;
        *reinterpret_cast<f32x4*>(o) = a;
        *reinterpret_cast<f32x4*>(o + 4) = b;
    }
    if (dbias != nullptr && blockIdx.y == 0) {
        const int rb = min(max(offsets[e], 0), TK);
        const int re = min(max(offsets[e + 1], rb), TK);
        __shared__ float part[kRbThreads];
        float sum = 0.f;
        for (int r = rb + (int)threadIdx.x; r < re; r += kRbThreads) sum += dk_perm[r];
        part[threadIdx.x] = sum;
        __syncthreads();
        for (int h = kRbThreads / 2; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) dbias[e] = part[0];
    }
}

}  // namespace
}  // namespace moe

namespace {
int64_t rb_max_chunks(int64_t T, int32_t k, int32_t E) { return moe::cdiv<int64_t>(T * k, moe::kRbChunk) + E; }
}  // namespace

// dk per slot [T, k], dk per permuted row [T*k], chunk offsets [E+1], and the weight
// gradient's chunk partials [cdiv(T*k, kRbChunk) + E, d] fp32.
size_t moe_route_backward_workspace_bytes(int64_t T, int64_t d, int32_t E, int32_t k) {
    if (T < 0 || d <= 0 || E < 1 || k < 1) return 256;
    return 2 * moe::rb_align((size_t)T * k * 4) + moe::rb_align((size_t)(E + 1) * 4) +
           moe::rb_align((size_t)rb_max_chunks(T, k, E) * d * 4);
}

extern "C" moe_status_t moe_route_backward(const void* x, const void* w_router, int32_t dtype, const float* keys,
                                           const int32_t* topk_idx, const float* d_topk_w, const int32_t* offsets,
                                           const int32_t* row_of, const int32_t* src_token, int64_t T, int64_t d,
                                           int32_t E, int32_t k, int32_t score, float* d_keys_sel, void* d_x,
                                           int32_t accumulate_dx, const void* d_x_perm, const void* d_x_perm_shared,
                                           float* d_w_router, float* d_bias, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    if (T < 0 || d <= 0 || d % 8 != 0 || E < 1 || E > 256 || k < 1 || k > 16 || k > E) return MOE_EINVAL;
    if (T * (int64_t)k > ((int64_t)1 << 30) || d > INT32_MAX / 16 || T * (int64_t)d > ((int64_t)1 << 40))
        return MOE_EINVAL;
    if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    const bool want_w = d_w_router != nullptr || d_bias != nullptr;
    if (want_w && !offsets) return MOE_EINVAL;
    if (T == 0) {
        if (!want_w) return MOE_OK;
    } else {
        if (!keys || !topk_idx || !d_topk_w || !row_of) return MOE_EINVAL;
        if (d_x && (!w_router || !moe_aligned16(w_router) || !moe_aligned16(d_x))) return MOE_EINVAL;
        if (d_x_perm && (!d_x || !moe_aligned16(d_x_perm))) return MOE_EINVAL;
        if (d_x_perm_shared && (!d_x_perm || !moe_aligned16(d_x_perm_shared))) return MOE_EINVAL;
        if (want_w && (!x || !src_token || !moe_aligned16(x))) return MOE_EINVAL;
    }
    if (d_w_router && !moe_aligned16(d_w_router)) return MOE_EINVAL;
    if (!workspace || workspace_bytes < moe_route_backward_workspace_bytes(T, d, E, k)) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    const int Ti = (int)T, di = (int)d, TK = (int)(T * k);
    // the per-slot gradient goes straight to d_keys_sel when the caller wants it
    float* dk_sel = d_keys_sel != nullptr ? d_keys_sel : (float*)workspace;
    float* dk_perm = (float*)((char*)workspace + moe::rb_align((size_t)T * k * 4));
    const int esize = dtype == MOE_BF16 ? 2 : 4;
    if (T > 0) {
        hipLaunchKernelGGL(moe::route_bwd_keys_kernel, dim3((unsigned)moe::cdiv(Ti, moe::kRbThreads)),
                           dim3(moe::kRbThreads), 0, s, keys, topk_idx, d_topk_w, row_of, Ti, E, k, score, TK, dk_sel,
                           dk_perm);
        MOE_CHECK_LAUNCH();
        if (d_x != nullptr) {
            if (esize == 2)
                hipLaunchKernelGGL(moe::route_bwd_dx_kernel<2>, dim3((unsigned)Ti), dim3(moe::kRbThreads), 0, s,
                                   (const char*)w_router, topk_idx, dk_sel, di, E, k, accumulate_dx != 0 ? 1 : 0,
                                   (char*)d_x, (const char*)d_x_perm, (const char*)d_x_perm_shared, row_of, TK);
            else
                hipLaunchKernelGGL(moe::route_bwd_dx_kernel<4>, dim3((unsigned)Ti), dim3(moe::kRbThreads), 0, s,
                                   (const char*)w_router, topk_idx, dk_sel, di, E, k, accumulate_dx != 0 ? 1 : 0,
                                   (char*)d_x, (const char*)d_x_perm, (const char*)d_x_perm_shared, row_of, TK);
            MOE_CHECK_LAUNCH();
        }
    }
    if (want_w) {
        const int max_chunks = (int)rb_max_chunks(T, k, E);
        const int col_blocks = moe::cdiv(di, moe::kRbCols);
        int32_t* chunk_off = (int32_t*)((char*)dk_perm + moe::rb_align((size_t)T * k * 4));
        float* partial = (float*)((char*)chunk_off + moe::rb_align((size_t)(E + 1) * 4));
        hipLaunchKernelGGL(moe::route_bwd_chunks_kernel, dim3(1), dim3(moe::kRbThreads), 0, s, offsets, E, TK,
                           chunk_off);
        MOE_CHECK_LAUNCH();
        if (d_w_router != nullptr) {
            const dim3 grid((unsigned)max_chunks, (unsigned)col_blocks);
            if (esize == 2)
                hipLaunchKernelGGL(moe::route_bwd_dw_partial_kernel<2>, grid, dim3(moe::kRbThreads), 0, s,
                                   (const char*)x, offsets, chunk_off, src_token, dk_perm, Ti, di, E, TK, partial);
            else
                hipLaunchKernelGGL(moe::route_bwd_dw_partial_kernel<4>, grid, dim3(moe::kRbThreads), 0, s,
                                   (const char*)x, offsets, chunk_off, src_token, dk_perm, Ti, di, E, TK, partial);
            MOE_CHECK_LAUNCH();
        }
        hipLaunchKernelGGL(moe::route_bwd_dw_reduce_kernel, dim3((unsigned)E, (unsigned)col_blocks),
                           dim3(moe::kRbThreads), 0, s, partial, offsets, chunk_off, dk_perm, di, TK, max_chunks,
                           d_w_router, d_bias);
        MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
}

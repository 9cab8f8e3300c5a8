// moe_group_quant_mxfp8: MXFP8 block quantisation (E4M3 elements, one E8M0 scale per 32
// elements along a GEMM's contraction axis), row-wise or group-aware column-wise.
//
// [Blog] "Optimisations dropless MoE needs": the MXFP8 quantisation must be group-aware;
// [Reading] contribution 3: MoE low precision needs group quantisation and dynamic-shape
// alignment. [OCP-MX]: a block's shared exponent is floor(log2(amax)) - 8 (8 = E4M3's
// largest exponent), stored as an E8M0 byte (+127, clamped to 0..254); each element is
// rounded to nearest-even E4M3 after division by 2^exponent, saturating at +-448.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlock = 32;
constexpr int kGroupAlign = 4;   // column-wise: each group's blocks start on a multiple of 4 blocks (128 rows)

// Row of `in` that feeds logical row r: row_index[r] (clamped into the input) or r itself.
__device__ __forceinline__ int64_t in_row(const int32_t* row_index, int64_t in_rows, int64_t r) {
    if (!row_index) return r;
    const int64_t v = row_index[r];
    return v < 0 ? 0 : (v >= in_rows ? in_rows - 1 : v);
}

// E8M0 byte for a block whose largest magnitude is `amax` (0 for an all-zero block).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0u;
    int e2;
    (void)frexpf(amax, &e2);                  // amax = m * 2^e2, m in [0.5, 1)
    const int b = e2 - 1 - 8 + 127;
    return (uint32_t)min(max(b, 0), 254);
}

// 2^(127 - byte): the exact multiplier that divides by the block scale. byte <= 246 for any
// finite bf16/fp32 amax, so the result is a normal float.
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// Round a (scaled) value to E4M3 (OCP "FN": bias 7, 3 mantissa bits, subnormal step 2^-9,
// max 448, no infinities), nearest-even, saturating; returns the byte code (sign kept).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a >= 448.f) return sign | 0x7Eu;
    if (a < 0.015625f) {                       // below 2^-6: subnormal grid of step 2^-9
        return sign | (uint32_t)rintf(a * 512.f);   // 8 maps to 0x08, the smallest normal
    }
    // normal: round the 23-bit mantissa to 3 bits, nearest-even; a carry bumps the exponent
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t e = (u >> 23) - 127u + 7u;
    return sign | (e << 3) | ((u >> 20) & 7u);
}

__device__ __forceinline__ float load_val(const char* p, int esize) {
    return esize == 2 ? bf16_to_f32(*reinterpret_cast<const uint16_t*>(p)) : *reinterpret_cast<const float*>(p);
}

// Row-wise: one thread per 32-element block of a row; consecutive threads take consecutive
// blocks of a row so loads and code stores are contiguous.
template <int ESIZE>
__global__ __launch_bounds__(256) void quant_rows_kernel(const char* __restrict__ in, int64_t rows, int cols,
                                                         int64_t ld_in, const int32_t* __restrict__ row_index,
                                                         int64_t in_rows, uint8_t* __restrict__ q, int64_t ld_q,
                                                         uint8_t* __restrict__ sc, int64_t ld_sc) {
    const int nb = cols / kBlock;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * nb) return;
    const int64_t r = idx / nb;
    const int b = (int)(idx % nb);
    const char* src = in + (in_row(row_index, in_rows, r) * ld_in + (int64_t)b * kBlock) * ESIZE;
    float v[kBlock];
    if (ESIZE == 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[c * 8 + 2 * i] = __uint_as_float(w[i] << 16);
                v[c * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[c * 4 + i] = __uint_as_float(w[i]);
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t byte = mx_scale_byte(amax);
    const float inv = mx_inv_scale(byte);
    u32x4 out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= e4m3_code(v[h * 16 + w * 4 + i] * inv) << (8 * i);
            out[h][w] = word;
        }
    uint8_t* dst = q + r * ld_q + (int64_t)b * kBlock;
    *reinterpret_cast<u32x4*>(dst) = out[0];
    *reinterpret_cast<u32x4*>(dst + 16) = out[1];
    sc[r * ld_sc + b] = (uint8_t)byte;
}

// Group-aware column-wise, transposed output: block j (a global index over all groups'
// 32-row blocks) of column c covers rows [offsets[g] + 32 i, +32) of group g, where
// j = block_start[g] + i; its 32 codes go to q[c, 32 j ...] and its scale to sc[c, j].
// Group g owns 4 * ceil(m_g / 128) blocks, so every group starts on a 128-element boundary
// of the transposed rows (one K slice of the MXFP8 GEMM, with its 4 scale bytes in one
// aligned dword); blocks past the group's last row are all-zero (codes 0, scale byte 0).
__global__ __launch_bounds__(1024) void quant_block_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                                  int64_t rows, int32_t* __restrict__ block_start) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += 1024) {
        const int g = g0 + tid;
        int nb = 0;
        if (g < G) {
            const int b = (int)min<int64_t>(max(offsets[g], 0), rows);
            const int e = (int)min<int64_t>(max(offsets[g + 1], b), rows);
            nb = kGroupAlign * cdiv(e - b, kGroupAlign * kBlock);
        }
        int incl = nb;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int wbase = carry_s;
        for (int w = 0; w < wave; ++w) wbase += wsum[w];
        if (g < G) block_start[g] = wbase + incl - nb;
        __syncthreads();
        if (tid == 1023) carry_s = wbase + incl;
        __syncthreads();
    }
    if (tid == 0) block_start[G] = carry_s;
}

// One thread per (column, block); 64 consecutive columns per wave, so each of the 32 row
// reads of a wave is one contiguous segment.
template <int ESIZE>
__global__ __launch_bounds__(256) void quant_cols_kernel(const char* __restrict__ in, int64_t rows, int cols,
                                                         int64_t ld_in, const int32_t* __restrict__ row_index,
                                                         int64_t in_rows, const int32_t* __restrict__ offsets, int G,
                                                         const int32_t* __restrict__ block_start,
                                                         uint8_t* __restrict__ q, int64_t ld_q,
                                                         uint8_t* __restrict__ sc, int64_t ld_sc) {
    const int j = blockIdx.y;                       // global block index
    const int c = blockIdx.x * 256 + threadIdx.x;   // column
    if (j >= block_start[G] || c >= cols) return;
    int lo = 0, hi = G - 1;                          // group = last g with block_start[g] <= j
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (block_start[mid] <= j) lo = mid;
        else hi = mid - 1;
    }
    const int g = lo;
    const int gb = (int)min<int64_t>(max(offsets[g], 0), rows);
    const int ge = (int)min<int64_t>(max(offsets[g + 1], gb), rows);
    const int r0 = gb + (j - block_start[g]) * kBlock;
    const int n = max(0, min(kBlock, ge - r0));      // rows of this block (partial or none at a group's end)
    float v[kBlock];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
        v[i] = (i < n) ? load_val(in + (in_row(row_index, in_rows, r0 + i) * ld_in + c) * ESIZE, ESIZE) : 0.f;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const uint32_t byte = mx_scale_byte(amax);
    const float inv = mx_inv_scale(byte);
    u32x4 out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= e4m3_code(v[h * 16 + w * 4 + i] * inv) << (8 * i);
            out[h][w] = word;
        }
    uint8_t* dst = q + (int64_t)c * ld_q + (int64_t)j * kBlock;
    *reinterpret_cast<u32x4*>(dst) = out[0];
    *reinterpret_cast<u32x4*>(dst + 16) = out[1];
    sc[(int64_t)c * ld_sc + j] = (uint8_t)byte;
}

}  // namespace
}  // namespace moe

size_t moe_quant_workspace_bytes(int32_t G) { return ((size_t)(G < 1 ? 1 : G) + 1) * 4 + 255 & ~size_t(255); }

extern "C" moe_status_t moe_group_quant_mxfp8(const void* in, int32_t dtype, int64_t rows, int64_t cols,
                                              int64_t ld_in, const int32_t* row_index, int64_t in_rows,
                                              const int32_t* group_offsets, int32_t G, int32_t axis,
                                              uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_scales,
                                              int32_t* block_start, void* workspace, size_t workspace_bytes,
                                              void* stream) {
    if (rows < 0 || cols <= 0 || cols % moe::kBlock != 0 || cols > INT32_MAX / 2 || ld_in < cols) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (axis != 0 && axis != 1) return MOE_EINVAL;
    if (!row_index) in_rows = rows;
    else if (in_rows <= 0 && rows > 0) return MOE_EINVAL;
    const int esize = dtype == MOE_BF16 ? 2 : 4;
    hipStream_t s = (hipStream_t)stream;
    if (axis == 0) {
        if (rows == 0) return MOE_OK;
        if (!in || !q || !scales || ld_q < cols || ld_scales < cols / moe::kBlock) return MOE_EINVAL;
        if (!moe_aligned16(in) || !moe_aligned16(q) || (ld_in * esize) % 16 != 0 || ld_q % 16 != 0) return MOE_EINVAL;
        const int64_t n = rows * (cols / moe::kBlock);
        const dim3 grid((unsigned)moe::cdiv<int64_t>(n, 256));
        if (esize == 2)
            hipLaunchKernelGGL(moe::quant_rows_kernel<2>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                               row_index, in_rows, q, ld_q, scales, ld_scales);
        else
            hipLaunchKernelGGL(moe::quant_rows_kernel<4>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                               row_index, in_rows, q, ld_q, scales, ld_scales);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // axis 1: group-aware blocks of rows, transposed output
    if (G < 1 || !group_offsets || rows > INT32_MAX / 2) return MOE_EINVAL;
    // blocks over all groups, upper bound: sum_g 4 ceil(m_g / 128) <= 4 (ceil(rows / 128) + G)
    const int64_t nblk_cap = moe::kGroupAlign * (moe::cdiv<int64_t>(rows, moe::kGroupAlign * moe::kBlock) + G);
    if (!workspace && !block_start) return MOE_EWORKSPACE;
    if (!block_start && workspace_bytes < moe_quant_workspace_bytes(G)) return MOE_EWORKSPACE;
    if (!q || !scales || ld_q < nblk_cap * moe::kBlock || ld_scales < nblk_cap) return MOE_EINVAL;
    if (rows > 0 && !in) return MOE_EINVAL;
    if (!moe_aligned16(q) || ld_q % 16 != 0) return MOE_EINVAL;
    int32_t* bs = block_start ? block_start : (int32_t*)workspace;
    hipLaunchKernelGGL(moe::quant_block_prefix_kernel, dim3(1), dim3(1024), 0, s, group_offsets, G, rows, bs);
    MOE_CHECK_LAUNCH();
    if (rows == 0) return MOE_OK;
    const dim3 grid((unsigned)moe::cdiv<int64_t>(cols, 256), (unsigned)nblk_cap);
    if (esize == 2)
        hipLaunchKernelGGL(moe::quant_cols_kernel<2>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, group_offsets, G, bs, q, ld_q, scales, ld_scales);
    else
        hipLaunchKernelGGL(moe::quant_cols_kernel<4>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, group_offsets, G, bs, q, ld_q, scales, ld_scales);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

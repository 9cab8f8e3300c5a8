// moe_group_quant_mxfp8: MXFP8 block quantisation (E4M3 elements, one E8M0 scale per 32
// elements along a GEMM's contraction axis), row-wise or group-aware column-wise.
//
// [Blog] "Optimisations dropless MoE needs": the MXFP8 quantisation must be group-aware;
// [Reading] contribution 3: MoE low precision needs group quantisation and dynamic-shape
// alignment. [OCP-MX]: a block's shared exponent is floor(log2(amax)) - 8 (8 = E4M3's
// largest exponent), stored as an E8M0 byte (+127, clamped to 0..254); each element is
// rounded to nearest-even E4M3 after division by 2^exponent, saturating at +-448.
#include "moe_internal.h"
#include "swiglu_math.h"
#include "round_math.h"
#include "mx_math.h"

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
            const float* e = v + h * 16 + w * 4;
            out[h][w] = pack4_e4m3(e[0] * inv, e[1] * inv, e[2] * inv, e[3] * inv);
        }
    uint8_t* dst = q + r * ld_q + (int64_t)b * kBlock;
    *reinterpret_cast<u32x4*>(dst) = out[0];
    *reinterpret_cast<u32x4*>(dst + 16) = out[1];
    sc[r * ld_sc + b] = (uint8_t)byte;
}

// ---- MXFP4 ([OCP-MX] FP4 E2M1 elements: bias 1, one mantissa bit, values 0, 0.5, 1, 1.5, 2,
// 3, 4, 6; the block's shared exponent floor(log2 amax) - 2, 2 being E2M1's largest exponent)

// Row-wise MXFP4: one thread per 32-element block; the block's 32 codes go out as 16 bytes
// (two per byte, the even element in the low nibble), its scale as one byte.
template <int ESIZE>
__global__ __launch_bounds__(256) void quant_rows_fp4_kernel(const char* __restrict__ in, int64_t rows, int cols,
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
    const uint32_t byte = mx4_scale_byte(amax);
    const float inv = mx_inv_scale(byte);     // exact: the scaled values are v * 2^(127 - byte)
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(v[w * 8 + i] * inv) << (4 * i);
        out[w] = word;
    }
    *reinterpret_cast<u32x4*>(q + r * ld_q + (int64_t)b * (kBlock / 2)) = out;
    sc[r * ld_sc + b] = (uint8_t)byte;
}

// Group-aware column-wise, transposed, group-major output: group g owns nb_g = 4 ceil(m_g/128)
// blocks j = block_start[g] + i (i < nb_g) of 32 of its rows; its codes form a [cols, 32 nb_g]
// matrix at q + 32 cols block_start[g] (block i of column c at column offset 32 i) and its
// scales a [cols, nb_g] matrix at sc + cols block_start[g]. Each group thus starts on a
// 128-element boundary (one K slice of the MXFP8 GEMM, its 4 scale bytes one aligned dword),
// and one group's transposed block is contiguous in memory; blocks past the group's last row
// are all-zero (codes 0, scale byte 0).
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

// Column-wise tile: one workgroup quantises a 4-block chunk (128 rows of one group: every
// group starts on a multiple of 4 blocks) by kColTile columns. The rows are loaded with
// coalesced 16-byte loads into LDS (read through row_index when given); then each thread takes
// one block of two adjacent columns (one 4-byte LDS read per row; fp32: one block of one
// column): their maxima, scale bytes and codes. The codes are staged back
// in LDS transposed, so that the stores write each column's 128 bytes of the group's
// transposed block as one full line (8 lanes x 16 bytes) and its 4 scale bytes as one dword
// (16-byte pieces of 64 different lines per store instruction measured ~30% slower). A 34 KiB tile
// keeps several workgroups resident per CU, so one's loads overlap another's arithmetic.
// With q_row given, the same tile also yields the row-wise copy (blocks of 32 along each of
// its valid rows, at the logical row index): both layouts from one read of the input. LDS
// rows are padded by 16 bytes so that the row-wise pass's 16-byte reads of 16 rows at one
// column offset land on distinct banks.
constexpr int kColTile = 128;        // columns per workgroup (bf16; 64 for fp32)
#ifndef MOE_QUANT_XCD
#define MOE_QUANT_XCD 1               // XCD-aware tile order of the column-wise / dual pass (rows in place)
#endif
#ifndef MOE_QUANT_NT
#define MOE_QUANT_NT 1                // E4M3 code stores of the column-wise / dual pass non-temporal
                                      // (DeepSeek-V3 weight stacks 9.85 -> 9.62 ms)
#endif
// Which tile a workgroup of the column-wise grid (x: column tiles, y: 4-block chunks) takes.
// The hardware deals workgroups round-robin over the 8 XCDs in launch order. Every row's
// row-wise scale bytes of 8 consecutive column tiles (1,024 bf16 columns) share one 32-byte
// sector, and a column's chunk scales sit next to those of the chunks around it, so when the
// tiles writing one sector run on different XCDs, each L2 writes its few bytes back as a
// partial sector. Each XCD therefore takes one contiguous run of tiles, ordered by bands of 8
// column tiles, then by chunk, then by column tile inside the band: the 8 writers of a row's
// sector run back to back on one L2, and a column's neighbouring chunks 8 workgroups apart.
// Grids whose column tiles are not a multiple of 8 keep the launch order. Measured on the
// DeepSeek-V3 weight stacks: bytes written 17.35 -> 15.62 GB (algorithmic 15.57) for W_gate/up
// and 8.63 -> 7.79 GB for W_down, the two dual passes 9.05 -> 8.75 ms.
__device__ __forceinline__ void quant_tile_of_block(int& cx, int& cy) {
    const int X = (int)gridDim.x, Y = (int)gridDim.y;
    if (X % 8 != 0) {
        cx = (int)blockIdx.x;
        cy = (int)blockIdx.y;
        return;
    }
    const int L = (int)blockIdx.y * X + (int)blockIdx.x;       // launch order
    const int lam = (L % 8) * (X / 8 * Y) + L / 8;              // XCD L % 8 takes a contiguous run
    const int band = lam / (8 * Y), rem = lam % (8 * Y);
    cy = rem / 8;
    cx = band * 8 + rem % 8;
}

// SWB: the input is not read as such but formed while loading: the SwiGLU backward's
// dgu = [dg | du] (cols = 2f) from dh [rows, f] (`in`, ld_in) and the saved gate/up
// pre-activations gu [rows, 2f] (ld_gu), each value rounded to bf16 as moe_swiglu_backward
// stores it, so the codes equal those of quantising that kernel's output (f % 128 == 0: a
// tile lies in one half).
template <int ESIZE, bool SWB = false>
__global__ __launch_bounds__(256) void quant_cols_kernel(const char* __restrict__ in, int64_t rows, int cols,
                                                         int64_t ld_in, const int32_t* __restrict__ row_index,
                                                         int64_t in_rows, const int32_t* __restrict__ offsets, int G,
                                                         const int32_t* __restrict__ block_start,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                         uint8_t* __restrict__ q_row, int64_t ld_q_row,
                                                         uint8_t* __restrict__ s_row, int64_t ld_s_row,
                                                         const char* __restrict__ gu = nullptr, int64_t ld_gu = 0,
                                                         int f = 0, const float* __restrict__ row_scale = nullptr) {
    static_assert(!SWB || ESIZE == 2, "the fused SwiGLU-backward mode reads bf16");
    constexpr int TC = ESIZE == 2 ? kColTile : kColTile / 2;    // columns of this tile
    constexpr int PITCH = TC * ESIZE + 16;                       // LDS bytes per row (256 + pad)
    __shared__ __attribute__((aligned(16))) char tile[kGroupAlign * kBlock * PITCH];   // 34 KiB
    // rows read in place take the XCD-aware order; gathered rows keep the launch order, which
    // measured faster for them (the dY and x passes: 0.54 vs 0.57 ms, 0.275 vs 0.29 ms)
    int tx = (int)blockIdx.x, ty = (int)blockIdx.y;
    if (MOE_QUANT_XCD && row_index == nullptr) quant_tile_of_block(tx, ty);
    const int j = ty * kGroupAlign;                              // first block of the chunk
    const int c0 = tx * TC;
    const int t = threadIdx.x;
    if (j >= block_start[G]) return;                             // uniform over the workgroup
    int lo = 0, hi = G - 1;                                      // group = last g with block_start[g] <= j
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (block_start[mid] <= j) lo = mid;
        else hi = mid - 1;
    }
    const int g = lo;
    const int gb = (int)min<int64_t>(max(offsets[g], 0), rows);
    const int ge = (int)min<int64_t>(max(offsets[g + 1], gb), rows);
    const int jb = j - block_start[g];                          // block index inside the group
    const int nbg = block_start[g + 1] - block_start[g];        // the group's blocks (row stride / 32)
    const int r0 = gb + jb * kBlock;
    const int n = max(0, min(kGroupAlign * kBlock, ge - r0));   // valid rows of the chunk
    // load: 128 rows x 256 bytes in 16-byte pieces (rows past n and columns past the matrix
    // read as zero; the 16 pad bytes of each LDS row are never read). A thread's 8 loads are
    // all issued before the first LDS write, so 8 are in flight per lane instead of one.
    constexpr int PR = TC * ESIZE / 16;                          // 16-byte pieces per tile row
    constexpr int RS = 256 / PR;                                 // rows per pass of the workgroup
    constexpr int NL = kGroupAlign * kBlock / RS;                // rows (pieces) per thread
    static_assert(NL * RS == kGroupAlign * kBlock, "whole rows per thread");
    const int ncols = min(TC, cols - c0);
    const int pc = t % PR, i0 = t / PR;                          // this thread's piece column and first row
    const bool col_ok = pc * 16 < ncols * ESIZE;
    // every load reads a valid address (row and piece clamped into the matrix) and is issued
    // unconditionally, so all NL are in flight together; pieces outside the chunk become zero
    const int pc_safe = min(pc, ncols * ESIZE / 16 - 1);
    int64_t roff[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) roff[u] = min<int64_t>(r0 + i0 + u * RS, rows - 1);
    // scaled-gather mode: logical row r's values are row_scale[r] * in[row r], one rounding
    float rsc[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) rsc[u] = row_scale != nullptr ? row_scale[roff[u]] : 1.0f;
    if (row_index != nullptr) {   // gathered rows: all index loads first, then the clamps
        int32_t ix[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u) ix[u] = row_index[roff[u]];
#pragma unroll
        for (int u = 0; u < NL; ++u) roff[u] = min<int64_t>(max(ix[u], 0), in_rows - 1);
    }
    u32x4 lv[NL];
    u32x4 lv_up[SWB ? NL : 1];
    if constexpr (SWB) {
        // this workgroup owns columns [c0, c0 + TC) of dh and g: both the gate tile (dgu columns
        // c0..) and the up tile (columns f + c0..) come from one read of dh, g and u, in two
        // batches of NL/2 pieces; each value is rounded to bf16 as moe_swiglu_backward stores it
        constexpr int NB = NL / 2;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            u32x4 hv[NB], gv[NB], uv[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int64_t r = roff[hb * NB + u];
                hv[u] = *reinterpret_cast<const u32x4*>(in + (r * ld_in + c0) * 2 + pc_safe * 16);
                gv[u] = *reinterpret_cast<const u32x4*>(gu + (r * ld_gu + c0) * 2 + pc_safe * 16);
                uv[u] = *reinterpret_cast<const u32x4*>(gu + (r * ld_gu + f + c0) * 2 + pc_safe * 16);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                u32x4 og, ou;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t pg = 0u, pu = 0u;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int sh = 16 * e;
                        const float hh = __uint_as_float(((hv[u][w] >> sh) & 0xFFFFu) << 16);
                        const float gg = __uint_as_float(((gv[u][w] >> sh) & 0xFFFFu) << 16);
                        const float uu = __uint_as_float(((uv[u][w] >> sh) & 0xFFFFu) << 16);
                        float dg, du;
                        swiglu_grad(hh, gg, uu, dg, du);
                        pg |= (uint32_t)f32_to_bf16(dg) << sh;
                        pu |= (uint32_t)f32_to_bf16(du) << sh;
                    }
                    og[w] = pg;
                    ou[w] = pu;
                }
                lv[hb * NB + u] = og;
                lv_up[hb * NB + u] = ou;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < NL; ++u)
            lv[u] = *reinterpret_cast<const u32x4*>(in + (roff[u] * ld_in + c0) * ESIZE + pc_safe * 16);
        if (row_scale != nullptr) {
#pragma unroll
            for (int u = 0; u < NL; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if (ESIZE == 2) {
                        const float lo = mul_round_odd(rsc[u], __uint_as_float(lv[u][w] << 16));
                        const float hi = mul_round_odd(rsc[u], __uint_as_float(lv[u][w] & 0xFFFF0000u));
                        lv[u][w] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                    } else {
                        lv[u][w] = __float_as_uint(rsc[u] * __uint_as_float(lv[u][w]));
                    }
                }
        }
    }
    // one pass per output tile: the tile's values go to LDS, then both copies are written
    // (the fused SwiGLU-backward mode makes a second pass for the up half's tile)
#pragma unroll 1
    for (int half = 0; half < (SWB ? 2 : 1); ++half) {
        const int c0o = c0 + half * f;                           // first output column of the tile
        if (half == 1) {
            __syncthreads();                                     // the first pass's stores have read LDS
#pragma unroll
            for (int u = 0; u < NL; ++u) lv[u] = lv_up[SWB ? u : 0];
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const bool ok = col_ok && i0 + u * RS < n;
#pragma unroll
            for (int w = 0; w < 4; ++w) lv[u][w] = ok ? lv[u][w] : 0u;
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) *reinterpret_cast<u32x4*>(tile + (i0 + u * RS) * PITCH + pc * 16) = lv[u];
        __syncthreads();
        if (q_row != nullptr) {
            // row-wise copy: unit u = (tile row u / HB, half block u % HB); the two lanes of a block
            // combine their maxima with one shuffle, and 8 consecutive lanes write 128 contiguous
            // bytes of one row (bf16; 4 lanes and 64 bytes for fp32)
            constexpr int HB = TC / 16;                              // half blocks per tile row
            constexpr int P16 = 16 * ESIZE / 16;                     // 16-byte LDS reads per half block
            static_assert((kGroupAlign * kBlock * HB) % 256 == 0, "whole waves per pass");
            for (int u = t; u < kGroupAlign * kBlock * HB; u += 256) {
                const int i = u / HB, hb = u % HB;
                const bool live = i < n && hb * 16 < ncols;          // same for both lanes of a block
                const char* src = tile + i * PITCH + hb * 16 * ESIZE;
                float v[16];
#pragma unroll
                for (int c = 0; c < P16; ++c) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 16);
                    if (ESIZE == 2) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[c * 8 + 2 * e] = __uint_as_float(w[e] << 16);
                            v[c * 8 + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[c * 4 + e] = __uint_as_float(w[e]);
                    }
                }
                float amax = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
                amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));      // the block's other half
                const uint32_t byte = mx_scale_byte(amax);
                const float inv = mx_inv_scale(byte);
                u32x4 out;
#pragma unroll
                for (int w = 0; w < 4; ++w) out[w] = pack4_e4m3(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv,
                                                                 v[4 * w + 3] * inv);
                if (live) {
                    const int64_t r = r0 + i;                        // logical row
                    u32x4* dst = reinterpret_cast<u32x4*>(q_row + r * ld_q_row + c0o + hb * 16);
                    if (MOE_QUANT_NT) __builtin_nontemporal_store(out, dst);
                    else *dst = out;
                    if ((hb & 1) == 0) s_row[r * ld_s_row + c0o / kBlock + hb / 2] = (uint8_t)byte;
                }
            }
        }
        // (column, block) units of this thread: bf16 threads read two adjacent columns with one
        // 4-byte LDS read per row and quantise one block of each; fp32 threads one block of one column
        constexpr int NU = kGroupAlign * TC / 256;                   // 2 bf16, 1 fp32
        int ucol[NU], ublk[NU];
        float v[NU][kBlock];
        if constexpr (ESIZE == 2) {
            const int cp = t % (TC / 2), b = t / (TC / 2);
#pragma unroll
            for (int i = 0; i < kBlock; ++i) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (b * kBlock + i) * PITCH + cp * 4);
                v[0][i] = __uint_as_float(w << 16);
                v[NU - 1][i] = __uint_as_float(w & 0xFFFF0000u);
            }
            ucol[0] = 2 * cp;
            ucol[NU - 1] = 2 * cp + 1;
            ublk[0] = ublk[NU - 1] = b;
        } else {
            const int col = t % TC, b = t / TC;
#pragma unroll
            for (int i = 0; i < kBlock; ++i) v[0][i] = *reinterpret_cast<const float*>(tile + (b * kBlock + i) * PITCH + col * 4);
            ucol[0] = col;
            ublk[0] = b;
        }
        // codes and scale bytes of the units, kept in registers until the tile is free
        u32x4 codes[NU][2];
        uint32_t sbytes[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
            const uint32_t byte = mx_scale_byte(amax);
            const float inv = mx_inv_scale(byte);
            sbytes[u] = byte;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float* e = v[u] + h * 16 + w * 4;
                    codes[u][h][w] = pack4_e4m3(e[0] * inv, e[1] * inv, e[2] * inv, e[3] * inv);
                }
        }
        // Stage the chunk's transposed codes in LDS (column c's 4 blocks = 128 contiguous bytes,
        // rows padded to 144 bytes) and its scale bytes (4 per column, one dword), then write
        // them out so that 8 consecutive lanes cover one column's full 128-byte line.
        constexpr int SP = kGroupAlign * kBlock + 16;               // staged bytes per column
        char* stage = tile;                                          // TC * SP <= the tile's size
        uint32_t* sstage = reinterpret_cast<uint32_t*>(tile + TC * SP);
        static_assert(TC * SP + TC * 4 <= kGroupAlign * kBlock * PITCH, "staging fits in the tile");
        __syncthreads();                                             // every thread is done reading the tile
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            char* d = stage + ucol[u] * SP + ublk[u] * kBlock;
            *reinterpret_cast<u32x4*>(d) = codes[u][0];
            *reinterpret_cast<u32x4*>(d + 16) = codes[u][1];
            reinterpret_cast<uint8_t*>(sstage)[ucol[u] * kGroupAlign + ublk[u]] = (uint8_t)sbytes[u];
        }
        __syncthreads();
        const int64_t gbase = (int64_t)cols * block_start[g];      // the group's transposed block
        constexpr int PIECES_OUT = TC * kGroupAlign * kBlock / 16;   // 16-byte pieces of the chunk
        for (int pcs = t; pcs < PIECES_OUT; pcs += 256) {
            const int cc = pcs / (kGroupAlign * kBlock / 16), ch = pcs % (kGroupAlign * kBlock / 16);
            if (cc >= ncols) continue;
            const int64_t c = c0o + cc;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + cc * SP + ch * 16);
            u32x4* dst = reinterpret_cast<u32x4*>(q + (gbase + c * nbg + jb) * kBlock + ch * 16);
            if (MOE_QUANT_NT) __builtin_nontemporal_store(v, dst);
            else *dst = v;
        }
        if (t < ncols) *reinterpret_cast<uint32_t*>(sc + gbase + (int64_t)(c0o + t) * nbg + jb) = sstage[t];
    }
}

// Weight of each permuted row for the combine's transpose: the routed row of (t, j) carries
// topk_w[t, j]; the shared expert's rows (T*k + t) carry 1.
__global__ __launch_bounds__(256) void row_weights_kernel(const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ row_of, int T, int k,
                                                          int shared, float* __restrict__ w_perm) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int TK = T * k;
    if (i < TK) w_perm[min(max(row_of[i], 0), TK - 1)] = topk_w[i];
    else if (shared && i < TK + T) w_perm[i] = 1.0f;
}

}  // namespace
}  // namespace moe

size_t moe_quant_workspace_bytes(int32_t G) { return ((size_t)(G < 1 ? 1 : G) + 1) * 4 + 255 & ~size_t(255); }

// Argument checks of the column-wise path, done before anything is enqueued.
static moe_status_t quant_colwise_check(const void* in, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_in,
                                        const int32_t* group_offsets, int32_t G, const uint8_t* q, int64_t ld_q,
                                        const uint8_t* scales, int64_t ld_scales, const int32_t* block_start,
                                        const void* workspace, size_t workspace_bytes) {
    const int esize = dtype == MOE_BF16 ? 2 : 4;
    if (G < 1 || !group_offsets || rows > INT32_MAX / 2) return MOE_EINVAL;
    // blocks over all groups, upper bound: sum_g 4 ceil(m_g / 128) <= 4 (ceil(rows / 128) + G)
    const int64_t nblk_cap = moe::kGroupAlign * (moe::cdiv<int64_t>(rows, moe::kGroupAlign * moe::kBlock) + G);
    if (!workspace && !block_start) return MOE_EWORKSPACE;
    if (!block_start && workspace_bytes < moe_quant_workspace_bytes(G)) return MOE_EWORKSPACE;
    // group-major output: the caller passes the capacity in blocks as ld_scales (and 32 times
    // it as ld_q): q holds 32 * cols * nblk bytes, scales cols * nblk bytes
    if (!q || !scales || ld_scales < nblk_cap || ld_q != 32 * ld_scales) return MOE_EINVAL;
    if (rows > 0 && !in) return MOE_EINVAL;
    if (!moe_aligned16(q)) return MOE_EINVAL;
    // 16-byte row loads and 4-byte scale words
    if ((reinterpret_cast<uintptr_t>(in) & 15) || (ld_in * esize) % 16 || (cols * esize) % 16) return MOE_EINVAL;
    if (reinterpret_cast<uintptr_t>(scales) & 3) return MOE_EINVAL;
    return MOE_OK;
}

// Shared host path of the column-wise mode (and of the dual mode when q_row is given).
static moe_status_t quant_colwise(const void* in, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_in,
                                  const int32_t* row_index, int64_t in_rows, const int32_t* group_offsets, int32_t G,
                                  uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_scales,
                                  uint8_t* q_row, int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row,
                                  int32_t* block_start, void* workspace, size_t workspace_bytes, hipStream_t s,
                                  const void* gu = nullptr, int64_t ld_gu = 0, int64_t f = 0,
                                  const float* row_scale = nullptr) {
    const int esize = dtype == MOE_BF16 ? 2 : 4;
    const moe_status_t chk = quant_colwise_check(in, dtype, rows, cols, ld_in, group_offsets, G, q, ld_q, scales,
                                                 ld_scales, block_start, workspace, workspace_bytes);
    if (chk != MOE_OK) return chk;
    const int64_t nblk_cap = moe::kGroupAlign * (moe::cdiv<int64_t>(rows, moe::kGroupAlign * moe::kBlock) + G);
    int32_t* bs = block_start ? block_start : (int32_t*)workspace;
    hipLaunchKernelGGL(moe::quant_block_prefix_kernel, dim3(1), dim3(1024), 0, s, group_offsets, G, rows, bs);
    MOE_CHECK_LAUNCH();
    if (rows == 0) return MOE_OK;
    const int tc = esize == 2 ? moe::kColTile : moe::kColTile / 2;
    // the fused SwiGLU-backward mode: one workgroup per TC columns of dh writes two tiles
    const dim3 grid((unsigned)moe::cdiv<int64_t>(gu != nullptr ? f : cols, tc), (unsigned)(nblk_cap / moe::kGroupAlign));
    if (gu != nullptr)
        hipLaunchKernelGGL((moe::quant_cols_kernel<2, true>), grid, dim3(256), 0, s, (const char*)in, rows, (int)cols,
                           ld_in, row_index, in_rows, group_offsets, G, bs, q, scales, q_row, ld_q_row, s_row,
                           ld_s_row, (const char*)gu, ld_gu, (int)f);
    else if (esize == 2)
        hipLaunchKernelGGL(moe::quant_cols_kernel<2>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, group_offsets, G, bs, q, scales, q_row, ld_q_row, s_row, ld_s_row,
                           nullptr, 0, 0, row_scale);
    else
        hipLaunchKernelGGL(moe::quant_cols_kernel<4>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, group_offsets, G, bs, q, scales, q_row, ld_q_row, s_row, ld_s_row,
                           nullptr, 0, 0, row_scale);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" moe_status_t moe_group_quant_mxfp8(const void* in, int32_t dtype, int64_t rows, int64_t cols,
                                              int64_t ld_in, const int32_t* row_index, int64_t in_rows,
                                              const int32_t* group_offsets, int32_t G, int32_t axis,
                                              uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_scales,
                                              int32_t* block_start, void* workspace, size_t workspace_bytes,
                                              void* stream) {
    if (rows < 0 || cols <= 0 || cols > INT32_MAX / 2 || ld_in < cols) return MOE_EINVAL;
    if (axis == 0 && cols % moe::kBlock != 0) return MOE_EINVAL;   // row-wise blocks run along cols
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
    return quant_colwise(in, dtype, rows, cols, ld_in, row_index, in_rows, group_offsets, G, q, ld_q, scales,
                         ld_scales, nullptr, 0, nullptr, 0, block_start, workspace, workspace_bytes, s);
}

extern "C" moe_status_t moe_group_quant_mxfp4(const void* in, int32_t dtype, int64_t rows, int64_t cols,
                                              int64_t ld_in, const int32_t* row_index, int64_t in_rows, uint8_t* q,
                                              int64_t ld_q, uint8_t* scales, int64_t ld_scales, void* stream) {
    if (rows < 0 || cols <= 0 || cols > INT32_MAX / 2 || ld_in < cols || cols % moe::kBlock != 0) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (!row_index) in_rows = rows;
    else if (in_rows <= 0 && rows > 0) return MOE_EINVAL;
    if (rows == 0) return MOE_OK;
    const int esize = dtype == MOE_BF16 ? 2 : 4;
    if (!in || !q || !scales || ld_q < cols / 2 || ld_scales < cols / moe::kBlock) return MOE_EINVAL;
    if (!moe_aligned16(in) || !moe_aligned16(q) || (ld_in * esize) % 16 != 0 || ld_q % 16 != 0) return MOE_EINVAL;
    const int64_t n = rows * (cols / moe::kBlock);
    const dim3 grid((unsigned)moe::cdiv<int64_t>(n, 256));
    hipStream_t s = (hipStream_t)stream;
    if (esize == 2)
        hipLaunchKernelGGL(moe::quant_rows_fp4_kernel<2>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, q, ld_q, scales, ld_scales);
    else
        hipLaunchKernelGGL(moe::quant_rows_fp4_kernel<4>, grid, dim3(256), 0, s, (const char*)in, rows, (int)cols, ld_in,
                           row_index, in_rows, q, ld_q, scales, ld_scales);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" moe_status_t moe_group_quant_mxfp8_dual(const void* in, int32_t dtype, int64_t rows, int64_t cols,
                                                   int64_t ld_in, const int32_t* row_index, int64_t in_rows,
                                                   const int32_t* group_offsets, int32_t G, uint8_t* q_row,
                                                   int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row,
                                                   uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col,
                                                   int64_t ld_s_col, int32_t* block_start, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
    if (rows < 0 || cols <= 0 || cols > INT32_MAX / 2 || ld_in < cols || cols % moe::kBlock != 0) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (!row_index) in_rows = rows;
    else if (in_rows <= 0 && rows > 0) return MOE_EINVAL;
    if (!q_row || !s_row || ld_q_row < cols || ld_s_row < cols / moe::kBlock) return MOE_EINVAL;
    if (!moe_aligned16(q_row) || ld_q_row % 16 != 0) return MOE_EINVAL;
    return quant_colwise(in, dtype, rows, cols, ld_in, row_index, in_rows, group_offsets, G, q_col, ld_q_col, s_col,
                         ld_s_col, q_row, ld_q_row, s_row, ld_s_row, block_start, workspace, workspace_bytes,
                         (hipStream_t)stream);
}

extern "C" moe_status_t moe_swiglu_backward_quant_mxfp8_dual(const void* dh, int64_t ld_dh, const void* gu,
                                                             int64_t ld_gu, int32_t dtype, int64_t rows, int64_t f,
                                                             const int32_t* group_offsets, int32_t G, uint8_t* q_row,
                                                             int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row,
                                                             uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col,
                                                             int64_t ld_s_col, int32_t* block_start, void* workspace,
                                                             size_t workspace_bytes, void* stream) {
    if (rows < 0 || f <= 0 || f % (moe::kColTile) != 0 || f > INT32_MAX / 4) return MOE_EINVAL;
    if (ld_dh < f || ld_gu < 2 * f || ld_dh % 8 != 0 || ld_gu % 8 != 0) return MOE_EINVAL;
    if (dtype != MOE_BF16) return MOE_ENOTSUP;
    if (rows > 0 && (!gu || !moe_aligned16(gu))) return MOE_EINVAL;
    const int64_t cols = 2 * f;
    if (!q_row || !s_row || ld_q_row < cols || ld_s_row < cols / moe::kBlock) return MOE_EINVAL;
    if (!moe_aligned16(q_row) || ld_q_row % 16 != 0) return MOE_EINVAL;
    return quant_colwise(dh, dtype, rows, cols, ld_dh, nullptr, rows, group_offsets, G, q_col, ld_q_col, s_col,
                         ld_s_col, q_row, ld_q_row, s_row, ld_s_row, block_start, workspace, workspace_bytes,
                         (hipStream_t)stream, gu, ld_gu, f);
}

size_t moe_combine_bwd_quant_workspace_bytes(int64_t T, int32_t k, int32_t G) {
    const int64_t rows = T > 0 ? T * (k > 0 ? k : 1) + T : 0;    // room for the shared rows
    return (((size_t)rows * 4 + 255) & ~size_t(255)) + moe_quant_workspace_bytes(G);
}

extern "C" moe_status_t moe_combine_backward_quant_mxfp8_dual(
    const void* d_out, int32_t dtype, const float* topk_w, const int32_t* row_of, const int32_t* src_token, int64_t T,
    int64_t d, int32_t k, int32_t shared_group, const int32_t* group_offsets, int32_t G, uint8_t* q_row,
    int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row, uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col,
    int64_t ld_s_col, int32_t* block_start, void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || d <= 0 || d % moe::kBlock != 0 || d > INT32_MAX / 2 || k < 1 || k > 16) return MOE_EINVAL;
    if (T * (int64_t)(k + 1) > INT32_MAX / 4) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (!workspace || workspace_bytes < moe_combine_bwd_quant_workspace_bytes(T, k, G)) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_EINVAL;
    if (T > 0 && (!d_out || !topk_w || !row_of || !src_token)) return MOE_EINVAL;
    if (!q_row || !s_row || ld_q_row < d || ld_s_row < d / moe::kBlock) return MOE_EINVAL;
    if (!moe_aligned16(q_row) || ld_q_row % 16 != 0) return MOE_EINVAL;
    const int64_t rows = T * k + (shared_group ? T : 0);
    const size_t wbytes = ((size_t)(T > 0 ? T * k + T : 0) * 4 + 255) & ~size_t(255);
    // every argument of the quantiser is checked before the row-weight kernel is enqueued
    const moe_status_t chk = quant_colwise_check(d_out, dtype, rows, d, d, group_offsets, G, q_col, ld_q_col, s_col,
                                                 ld_s_col, block_start, (char*)workspace + wbytes,
                                                 workspace_bytes - wbytes);
    if (chk != MOE_OK) return chk;
    float* w_perm = (float*)workspace;
    hipStream_t s = (hipStream_t)stream;
    if (rows > 0) {
        hipLaunchKernelGGL(moe::row_weights_kernel, dim3((unsigned)moe::cdiv<int64_t>(rows, 256)), dim3(256), 0, s,
                           topk_w, row_of, (int)T, k, shared_group ? 1 : 0, w_perm);
        MOE_CHECK_LAUNCH();
    }
    return quant_colwise(d_out, dtype, rows, d, d, src_token, T > 0 ? T : 1, group_offsets, G, q_col, ld_q_col, s_col,
                         ld_s_col, q_row, ld_q_row, s_row, ld_s_row, block_start, (char*)workspace + wbytes,
                         workspace_bytes - wbytes, s, nullptr, 0, 0, w_perm);
}

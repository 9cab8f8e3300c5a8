// moe_grouped_gemm: one launch computes every group's product at its real row count.
//
// [Blog] "Optimisation 1": a grouped GEMM runs all experts' matmuls in one kernel call, each
// at its actual token count, and computes only the regions that hold real tokens; the
// alternatives (a host loop over experts after a device-to-host copy of the counts, or a
// batched GEMM padded to the worst case) are what it replaces. [Blog] Figure 3 paragraph:
// the grouped MLP is two such GEMMs, gate/up then down. [Blog] "Optimisations dropless MoE
// needs": the expert GEMMs also run in MXFP8 ([OCP-MX] block-scaled E4M3).
//
// Design (gfx950):
//  * A one-workgroup schedule kernel turns the device-resident group offsets into a tile
//    prefix (tiles of group g start at tile_start[g]); the host never sees group sizes.
//  * Each group gets its own tile height BM in {16, 32, 64, 128} from its row count, so tiny
//    groups do not pay for 128-row tiles and empty groups get no tile at all.
//  * Persistent workgroups (one per CU: 8 MFMA waves + 4 load waves) walk the tile list; tiles are ordered group
//    by group, in supertiles of 4 column tiles x all row tiles, and handed out so the 32 CUs
//    of one XCD work on consecutive tiles (shared A/B panels hit that XCD's L2).
//  * bf16 launches whose A rows are read in order (no row index), with a bf16 output and no
//    G|U save, run gemm_split_kernel instead: 8-wave workgroups that take each large group's
//    full 256-row chunks as 256 x 256 tiles (every wave loads 64 operand rows per stage into a
//    two-stage ring) and the rest of the rows as the row tiles below, with the MFMA waves
//    issuing their own loads; outputs are bit-identical to the persistent kernel's.
//  * Operands stream global -> LDS with 16-byte DMA loads (no VGPR staging) through a 3-stage
//    ring of K slices (64 bf16 or 128 fp8 = 128 bytes per row). Four producer waves (one per
//    SIMD) issue every load and wait for it; the MFMA waves only read LDS and multiply, so
//    neither role holds the other's registers or stalls on the other's waits (measured 2-6%
//    faster than MFMA waves that also issue the loads). LDS rows are XOR-swizzled so
//    MFMA fragment reads are bank-conflict free; fragments are double-buffered in registers.
//  * bf16: v_mfma_f32_32x32x16_bf16 (16x16x32 for 16/32-row tiles). MXFP8: E4M3 codes with one
//    E8M0 scale per 32 K-elements; row tiles fetch each row's scales 16 bytes (4 MXFP8 or 2
//    MXFP4 stages) at a time into a two-slot scale ring, the weight-gradient tiles one dword (4
//    block scales) per row and stage, and v_mfma_scale_f32_32x32x64_f8f6f4 (16x16x128) applies
//    per-(row, 32-block) scales (the lane-to-block layout was measured; see the Mfma traits).
//    Accumulation is fp32 in both.
//  * The epilogue (optional SwiGLU) goes through LDS so that C is written in 16-byte chunks.
#include <algorithm>
#include <utility>

#include "moe_internal.h"
#include "mx_math.h"
#include "swiglu_math.h"

typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace moe {
namespace {

#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif
// 8 waves: two per SIMD, 64x64-ish wave tiles; 4 waves: one per SIMD with twice the wave tile
// (half the LDS fragment reads per MFMA), accumulators in the accumulation registers
#ifndef MOE_GEMM_PRODUCERS
#define MOE_GEMM_PRODUCERS 4      // extra waves that only issue the DMA loads (0: the MFMA waves do)
#endif
constexpr int kWaves = MOE_GEMM_WAVES;               // waves that hold accumulators
constexpr int kPWaves = MOE_GEMM_PRODUCERS;          // load-only waves
constexpr int kLWaves = kPWaves ? kPWaves : kWaves;  // waves that issue the DMA loads
constexpr int kThreads = (kWaves + kPWaves) * 64;
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 MFMA waves per workgroup");
constexpr int kBN = 256;          // B rows per tile (SwiGLU: 128 gate rows + 128 up rows)
constexpr int kRowBytes = 128;    // one LDS row per stage: 64 bf16 or 128 fp8 of K
constexpr int kChunks = kRowBytes / 16;
#ifndef MOE_GEMM_BUFFER_LDS
#define MOE_GEMM_BUFFER_LDS 1     // operand DMA through buffer_load ... lds (32-bit lane offsets, the
                                  // stage's K offset in a scalar) instead of global_load_lds:
                                  // measured 5-13% faster on the expert shapes (fewer VGPRs and
                                  // no per-load 64-bit address arithmetic)
#endif
// the buffer resource type and its builtins exist only in the device pass
#if MOE_GEMM_BUFFER_LDS && defined(__HIP_DEVICE_COMPILE__)
#define MOE_BUF_DMA 1
#else
#define MOE_BUF_DMA 0
#endif

#ifndef MOE_GEMM_SPLIT256
#define MOE_GEMM_SPLIT256 1       // bf16 groups' full 256-row chunks as 256 x 256 tiles (gemm_split_kernel)
#endif
// smallest group whose 256-row chunks take 256 x 256 tiles: K below MOE_GEMM_SPLIT_LONGK, and
// from it on. Measured on the DeepSeek-V3 group sizes (one MI355X; 257 groups, 73,728 rows):
// the down projection (K = 2,048) 2.96 -> 2.65 ms with every group of 256 rows or more split;
// the gate/up projection (K = 7,168) on unpermuted rows 5.47 ms unsplit, 5.58 / 5.48 / 5.35 ms
// with groups from 256 / 512 / 1,024 rows split. With gathered A rows (the fused gather) the
// gate/up projection ran 5.22 ms unsplit against 5.35-5.53 ms split at any threshold, so
// launches with a row index do not split.
#ifndef MOE_GEMM_SPLIT_MIN_ROWS
#define MOE_GEMM_SPLIT_MIN_ROWS 256
#endif
#ifndef MOE_GEMM_SPLIT_LONGK
#define MOE_GEMM_SPLIT_LONGK 4096
#endif
#ifndef MOE_GEMM_SPLIT_MIN_ROWS_LONGK
#define MOE_GEMM_SPLIT_MIN_ROWS_LONGK 1024
#endif
#ifndef MOE_GEMM_TILE256
#define MOE_GEMM_TILE256 0        // 256-row tiles for bf16 groups of >= 256 rows with a bf16 output (measured
                                  // slower on the DeepSeek-V3 and Mixtral shapes: longer tiles, worse tail)
#endif

// Operand formats of the MFMA path: bf16, E4M3 (MXFP8) and E2M1 (MXFP4, two per byte, the
// even element in the low nibble). A stage holds 128 bytes of every A and B row: 64 bf16,
// 128 E4M3 or 256 E2M1 values of K.
constexpr int kBF16 = 0, kE4M3 = 1, kE2M1 = 2;

// One LDS pipeline stage of a BM-row tile: BM A rows then kBN B rows of kRowBytes each, then
// (block-scaled formats) the E8M0 scale bytes of the stage's K slice per A row and per B row,
// as dwords: one per row for E4M3 (4 blocks of 32), two for E2M1 (8 blocks), dword h of every
// row together. A scale rows are loaded 64 per wave instruction, so their slot is rounded up
// to a multiple of 64 rows (a 16-row tile's scale load still writes 64 dwords and must not
// reach the B scales). Tiles up to 128 rows keep a 3-stage ring (a 4th stage for the 16/32-
// row tiles measured no faster on the expert shapes); 256-row tiles (64 KiB of operands per
// stage) fit two.
template <int BM, int FMT = kE4M3>
struct Stage {
    static constexpr int kScaleDw = FMT == kE2M1 ? 2 : 1;   // scale dwords per row and stage
    static constexpr int kScaleRowsA = (BM + 63) / 64 * 64;
    static constexpr int kData = (BM + kBN) * kRowBytes;
    static constexpr int kScaleA = kData;
    static constexpr int kScaleB = kData + kScaleRowsA * 4 * kScaleDw;
    static constexpr int kBytes = kData + (kScaleRowsA + kBN) * 4 * kScaleDw;
    static constexpr int kCount = BM == 256 ? 2 : 3;
};
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kPipeBytes = cmax(3 * Stage<128>::kBytes, 2 * Stage<256>::kBytes);   // 148.5 KiB
constexpr int kMaxGroups = 2047;
constexpr int kLdsBytes = kPipeBytes + (kMaxGroups + 1) * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
// Block-scaled row tiles (MXFP8, MXFP4; not the ragged-K mode) keep their scales out of the
// stages, in a ring of two batch slots: a batch holds 16 scale bytes (4 dwords, the scales of
// 4 MXFP8 or 2 MXFP4 stages) of every A and B row, 16 bytes per row, and is fetched by 4-byte
// DMA lanes of which 4 consecutive ones read one row's 16 contiguous bytes. One scale
// instruction thus covers 16 rows of a whole batch in 16 line requests, where a per-stage
// dword per row took 64 rows of one stage in 64. The operand stages then hold codes only (3 x 48 KiB),
// the two slots 12 KiB, which leaves room for a tile prefix of 1024 entries.
constexpr int kScBatchBytes = 16;                                   // scale bytes per row and batch
constexpr int kScSlot = (Stage<128>::kScaleRowsA + kBN) * kScBatchBytes;   // 6 KiB (largest BM)
constexpr int kMxData = 3 * Stage<128>::kData;                      // 144 KiB of operand stages
constexpr int kMxPipe = kMxData + 2 * kScSlot;                      // 156 KiB
template <int FMT>
constexpr int pipe_bytes() { return FMT == kBF16 ? kPipeBytes : kMxPipe; }
// groups of the row-tile schedule whose prefix fits past the ring (the ragged-K mode has no
// schedule and takes up to kMaxGroups)
template <int FMT>
constexpr int max_groups() { return FMT == kBF16 ? kMaxGroups : (160 * 1024 - kMxPipe) / 4 - 1; }
template <int FMT>
constexpr int lds_bytes() { return pipe_bytes<FMT>() + (max_groups<FMT>() + 1) * 4; }
static_assert(lds_bytes<kE4M3>() <= 160 * 1024 && max_groups<kE4M3>() == 1023, "block-scaled LDS budget");
static_assert(lds_bytes<kE4M3>() >= kPipeBytes + 8 * 1024, "the ragged-K stream's ring and staging fit");
constexpr int kSuper = 4;         // column tiles per supertile
// Ragged-K (weight-gradient) tiles write a 128 x 256 bf16 block each over a short K range, so
// output stores weigh more than operand reuse: with 16 or more column tiles they take wider
// supertiles (16 columns; measured on the DeepSeek-V3-shaped step: 6.59 -> 5.86 ms for the
// 28-column dW_gate/up, where 8 / 32 columns gave 5.95 / 6.15 ms and 2 gave 6.71 ms); narrower
// outputs keep kSuper (4 beat 2 and 8 on the 8-column dW_down).
constexpr int kSuperRK = 16;
constexpr int kSuperRKMinNT = 16;
#ifndef MOE_GEMM_C_NT
#define MOE_GEMM_C_NT 2           // ragged-row C stores non-temporal: 0 never, 1 without SwiGLU (outputs
                                  // the next kernel streams once; GEMM 2 at DeepSeek-V3 size -1.3%), 2 always
                                  // (H too, 302 MB at DeepSeek-V3 size, more than the MALL holds: GEMM 1
                                  // 5.12 -> 5.09 ms, GEMM 2 2.74 -> 2.75, forward 8.14 -> 8.12 ms)
#endif
#ifndef MOE_GEMM_RK_C_NT
#define MOE_GEMM_RK_C_NT 1        // weight-gradient (ragged-K) outputs stored non-temporally (never re-read
                                  // here; DeepSeek-V3 dW_gate/up 5.87 -> 5.52 ms, dW_down 2.84 -> 2.71 ms)
#endif
#ifndef MOE_GEMM_MX_FRAG_DB
#define MOE_GEMM_MX_FRAG_DB 1     // MXFP8 operand fragments double-buffered in registers like bf16 ones
#endif
#ifndef MOE_GEMM_RK_STREAM
#define MOE_GEMM_RK_STREAM 1      // ragged-K bf16-output tiles as one stream of K slices (gemm_rk_stream)
#endif

// 16-byte chunk c of LDS row r lives at slot c ^ swz(r). Measured on gfx950 with 128-byte
// rows: this XOR keeps ds_read_b128 of 16x16 and 32x32 MFMA fragments (16 or 32 rows at one
// chunk) bank-conflict free (~230 B/clk/CU), where c ^ (r & 7) conflicts 2-way for 32 rows.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ int bm_of_rows(int m) { return m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : 128; }

// Row tiles of a group of m rows: groups of up to 128 rows get one tile of 16/32/64/128 rows;
// larger groups get full 256-row tiles (when allowed), then full 128-row tiles, then one tile
// of 16/32/64/128 rows for what is left, so only the last tile carries padding rows.
struct RowTiles {
    int n256, n128, last;   // last: height of the final partial tile (0 = none)
    __device__ int count() const { return n256 + n128 + (last > 0 ? 1 : 0); }
};

__device__ __forceinline__ RowTiles row_tiles(int m, bool allow256) {
    RowTiles t{0, 0, 0};
    if (m <= 128) {
        t.last = m > 0 ? bm_of_rows(m) : 0;
        return t;
    }
    int rest = m;
    if (allow256 && m >= 256) {
        t.n256 = m / 256;
        rest -= 256 * t.n256;
    }
    t.n128 = rest / 128;
    rest -= 128 * t.n128;
    t.last = rest > 0 ? bm_of_rows(rest) : 0;
    return t;
}

// row tile mt of the decomposition -> first row inside the group and tile height
__device__ __forceinline__ void row_tile(const RowTiles& t, int mt, int& r_off, int& bm) {
    if (mt < t.n256) {
        r_off = 256 * mt;
        bm = 256;
    } else if (mt < t.n256 + t.n128) {
        r_off = 256 * t.n256 + 128 * (mt - t.n256);
        bm = 128;
    } else {
        r_off = 256 * t.n256 + 128 * t.n128;
        bm = t.last;
    }
}

// Rows of a group of m rows that 256 x 256 tiles cover (its full 256-row chunks) when the
// launch splits; its other row tiles start that many rows in.
// split_min: the smallest group that gets them (0: the launch does not split; else >= 256).
__device__ __forceinline__ int chunk256_rows(int m, int split_min) { return (split_min && m >= split_min) ? (m & ~255) : 0; }

// Rows [begin, end) of group g, clamped into [0, M] so that inconsistent offsets can never
// send a load or store outside the buffers.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int g, int M, int& begin, int& end) {
    begin = min(max(offsets[g], 0), M);
    end = min(max(offsets[g + 1], begin), M);
}

struct GemmParams {
    const int32_t* offsets;
    int G;
    int M;          // rows of C (row indices are clamped to it)
    int N;          // output columns
    int K;          // contraction length (elements)
    int NT;         // column tiles per group
    const char* A;  // all strides below are in elements of the operand's dtype
    int64_t lda;
    int64_t A_rows;
    const int32_t* a_rows;
    const char* B;
    int64_t ldb;
    int64_t b_stride;
    char* C;
    int64_t ldc;
    int c_f32;
    char* aux;
    int64_t ld_aux;
    const uint8_t* a_scale;   // MXFP8 only: E8M0 bytes [A_rows, K/32]
    int64_t lda_scale;
    const uint8_t* b_scale;   // group g: [N_B, K/32] at b_scale + g * b_scale_stride
    int64_t ldb_scale;
    int64_t b_scale_stride;
    const int32_t* tile_start;   // [G+1] in workspace (ragged rows): first tile of schedule position p
    const int32_t* order;        // [G] in workspace: group at schedule position p
    int allow256;                // ragged rows: 256-row tiles allowed (not for fp32 C)
    int64_t c_stride;            // ragged K: elements between groups' C
    int MT;                      // ragged K: row tiles per group
    // uniform groups (internal, 0 = off): group g owns C rows [g R, (g+1) R), its A rows are
    // A + (r - g R) * lda + g * a_group_stride (the K slices of one matrix), and no offsets,
    // row index or schedule are read
    int uniform_rows;
    int64_t a_group_stride;
    // fused output quantisation (ragged rows, bf16 C; 0 = off): the epilogue quantises the
    // bf16-rounded tile it writes, row-wise into q_row / s_row and (E4M3, when q_col is given)
    // group-aware column-wise into q_col / s_col at the blocks q_bs gives each group
    int q_fmt;                   // 0, kE4M3 or kE2M1
    uint8_t* q_row;
    int64_t ld_q_row;            // bytes
    uint8_t* s_row;
    int64_t ld_s_row;
    uint8_t* q_col;
    uint8_t* s_col;
    const int32_t* q_bs;         // [G+1] column-wise block prefix, written by the schedule kernel
    int64_t q_col_blocks;        // capacity of q_col / s_col in blocks
    int c_skip;                  // C is not written (only its quantised copies)
    int swb;                     // SwiGLU-backward epilogue: C = [dg | du] from dh and the saved aux
    // bf16 ragged rows (0 = off): the full 256-row chunks of every group of at least split256
    // rows are 256 x 256 tiles, its first tiles in the schedule; the rows past them get the
    // usual row tiles (gemm_split_kernel)
    int split256;
};

// ---------------------------------------------------------------------------------------
// schedule: the order in which the persistent workgroups take the groups' tiles.
//
// Groups of up to 128 rows are one row of tiles that stream their weights once (HBM-bound);
// larger groups are MFMA-bound. Taking them in expert order makes the chip alternate between
// phases that saturate HBM and phases that leave it idle, so the two classes are merged in
// proportion instead: every non-empty group gets the fraction of its class's tiles completed
// at its midpoint, and groups are taken in that order (ties: the larger class first, then by
// id). order[p] is the group at position p, tile_start[p] the first tile of that position;
// empty groups go last with no tiles. G <= 2047, one workgroup.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets, int G, int M,
                                                             int NT, int allow256, int32_t* __restrict__ tile_start,
                                                             int32_t* __restrict__ order,
                                                             int32_t* __restrict__ block_start = nullptr,
                                                             int split256 = 0) {
    __shared__ unsigned long long key[2048];
    __shared__ int tiles_of[2048];
    __shared__ int sorted[2048];
    __shared__ unsigned long long wsum[16];
    __shared__ unsigned long long carry_s;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // tiles per group, and each group's exclusive prefix of tiles within its class: one scan of
    // (small-class tiles << 32 | large-class tiles)
    unsigned long long pre[2];
    int rows_of[2] = {0, 0};   // this thread's groups' row counts (offsets are read once)
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int h = 0; h < 2; ++h) {
        const int g = h * 1024 + tid;
        int t = 0, small = 0;
        if (g < G) {
            int b, e;
            group_rows(offsets, g, M, b, e);
            rows_of[h] = e - b;
            // split: the full 256-row chunks' tiles, then the rest's
            const int c256 = chunk256_rows(e - b, split256);
            t = (c256 / 256 + row_tiles(e - b - c256, allow256 != 0).count()) * NT;
            small = (e - b) <= 128;
        }
        if (g < 2048) tiles_of[g] = t;
        const unsigned long long v = small ? ((unsigned long long)t << 32) : (unsigned long long)t;
        unsigned long long incl = v;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const unsigned long long o = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        unsigned long long base = carry_s;
        for (int w = 0; w < wave; ++w) base += wsum[w];
        pre[h] = base + incl - v;
        __syncthreads();
        if (tid == 1023) carry_s = base + incl;
        __syncthreads();
    }
    const unsigned long long tot = carry_s;
    const unsigned long long tot_small = tot >> 32, tot_large = tot & 0xFFFFFFFFull;
    for (int h = 0; h < 2; ++h) {
        const int g = h * 1024 + tid;
        unsigned long long k = ~0ull;   // padding and empty groups sort last
        if (g < G && tiles_of[g] > 0) {
            const int m = rows_of[h];
            const bool small = m <= 128;
            const unsigned long long p = small ? (pre[h] >> 32) : (pre[h] & 0xFFFFFFFFull);
            const unsigned long long total = small ? tot_small : tot_large;
            // midpoint fraction of the class's tiles in 2^-24 units
            const unsigned long long frac = ((2 * p + (unsigned long long)tiles_of[g]) << 23) / total;
            const bool first = small ? (tot_small >= tot_large) : (tot_large > tot_small);
            // groups cut into 256-row tiles (the longest tiles) go first, so the short tiles
            // of the other groups fill the end of the run instead of a long tile ending it
            const unsigned long long late = (allow256 != 0 && m >= 256) ? 0ull : 1ull;
            k = (late << 60) | (frac << 32) | ((unsigned long long)(first ? 0 : 1) << 16) | (unsigned long long)g;
        } else if (g < G) {
            k = (0xFFFFFFFull << 32) | (2ull << 60) | (unsigned long long)g;   // empty group: last, by id
        }
        key[g] = k;
    }
    __syncthreads();
    // ascending order by rank: the G keys are distinct (the group id is in the low bits), so a
    // key's position is the number of smaller keys; every thread counts them for its own keys
    // with broadcast LDS reads
    for (int h = 0; h < 2; ++h) {
        const int g = h * 1024 + tid;
        if (g < G) {
            const unsigned long long kg = key[g];
            int r = 0;
#pragma unroll 8
            for (int q = 0; q < G; ++q) r += key[q] < kg ? 1 : 0;
            sorted[r] = g;
        }
    }
    __syncthreads();
    // order and the tile prefix in schedule order
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int h = 0; h < 2; ++h) {
        const int p = h * 1024 + tid;
        int t = 0, g = 0;
        if (p < G) {
            g = sorted[p];
            t = tiles_of[g];
            order[p] = g;
        }
        int incl = t;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = (unsigned long long)incl;
        __syncthreads();
        int base = (int)carry_s;
        for (int w = 0; w < wave; ++w) base += (int)wsum[w];
        if (p < G) tile_start[p] = base + incl - t;
        __syncthreads();
        if (tid == 1023) carry_s = (unsigned long long)(base + incl);
        __syncthreads();
    }
    if (tid == 0) tile_start[G] = (int)carry_s;
    if (block_start == nullptr) return;
    // the column-wise quantisation's block prefix: group g owns 4 ceil(m_g / 128) blocks of 32
    // rows starting at block_start[g] (group order, the layout of moe_group_quant_mxfp8 axis 1)
    __syncthreads();
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int h = 0; h < 2; ++h) {
        const int g = h * 1024 + tid;
        int nb = 0;
        if (g < G) {
            int b, e;
            group_rows(offsets, g, M, b, e);
            nb = 4 * cdiv(e - b, 128);
        }
        int incl = nb;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = (unsigned long long)incl;
        __syncthreads();
        int base = (int)carry_s;
        for (int w = 0; w < wave; ++w) base += (int)wsum[w];
        if (g < G) block_start[g] = base + incl - nb;
        __syncthreads();
        if (tid == 1023) carry_s = (unsigned long long)(base + incl);
        __syncthreads();
    }
    if (tid == 0) block_start[G] = (int)carry_s;
}

// ---------------------------------------------------------------------------------------
// MFMA shapes. A lane's operand fragment is 16 bytes (bf16) or 32 bytes (fp8) of one row at
// consecutive K; `out_row/out_col` give the position of accumulator element r in the
// MS x MS output tile. Measured on MI355X from registers: 32x32x16 bf16 sustains ~2.28
// PFLOP/s with 8 accumulators, 16x16x32 at most ~1.95, so 64/128-row tiles use 32x32.
// ---------------------------------------------------------------------------------------
// f(integral_constant<L0 + i>) for i = 0 .. n-1, unrolled at compile time
template <int L0, int... Is, class F>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, L0 + Is>{}), ...);
}

template <int MS, int FMT>
struct Mfma;

template <>
struct Mfma<16, kBF16> {
    using acc_t = f32x4;
    static constexpr int KS = 2;                                    // k-steps per stage
    static constexpr int NACC = 4;
    static constexpr int kChunk2 = 0;                               // one 16-byte chunk
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 16; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 4 + lane / 16; }
    static constexpr __device__ __host__ int frag_block(int, int) { return 0; }   // no scales
    static __device__ __forceinline__ int out_row(int lane, int r) { return (lane / 16) * 4 + r; }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 16; }
};
template <>
struct Mfma<32, kBF16> {
    using acc_t = f32x16;
    static constexpr int KS = 4;
    static constexpr int NACC = 16;
    static constexpr int kChunk2 = 0;
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 32; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 2 + lane / 32; }
    static constexpr __device__ __host__ int frag_block(int, int) { return 0; }   // no scales
    static __device__ __forceinline__ int out_row(int lane, int r) { return (r / 4) * 8 + (lane / 32) * 4 + (r % 4); }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 32; }
};
// fp8 (measured on gfx950 with one-hot operands and distinct per-lane scales): a lane's 32
// bytes are two 16-byte K chunks that belong to two different MX blocks, and the scale a lane
// passes is applied to block `frag_block` of its row, whose two halves sit in this lane's
// and a partner lane's chunks. 32x32x64: lanes 32h+r hold K [16h, 16h+16) and [32+16h, ...),
// scale lane 32b+r owns block b. 16x16x128: lanes 16g+r hold K [16g, 16g+16) and
// [64+16g, ...), scale lane 16b+r owns block b. frag_chunk is the first chunk, the second
// follows kChunk2 chunks later.
template <>
struct Mfma<16, kE4M3> {
    using acc_t = f32x4;
    static constexpr int KS = 1;                                    // 16x16x128
    static constexpr int NACC = 4;
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 16; }
    static constexpr int kChunk2 = 4;
    static constexpr __device__ __host__ int frag_block(int lane, int ks) { return ks * 4 + lane / 16; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 8 + lane / 16; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (lane / 16) * 4 + r; }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 16; }
};
template <>
struct Mfma<32, kE4M3> {
    using acc_t = f32x16;
    static constexpr int KS = 2;                                    // 32x32x64
    static constexpr int NACC = 16;
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 32; }
    static constexpr int kChunk2 = 2;
    static constexpr __device__ __host__ int frag_block(int lane, int ks) { return ks * 2 + lane / 32; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 4 + lane / 32; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (r / 4) * 8 + (lane / 32) * 4 + (r % 4); }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 32; }
};
// fp4 (E2M1, measured on gfx950 with one-hot E2M1 operands against an E4M3 identity): a
// lane's 16 bytes are 32 consecutive K values of its row, the even one in the low nibble,
// i.e. one whole MX block, whose scale the lane passes. 32x32x64: lanes 32h+r hold K
// [32h, 32h+32); 16x16x128: lanes 16g+r hold K [32g, 32g+32). One 16-byte chunk per
// fragment, as for bf16.
template <>
struct Mfma<16, kE2M1> {
    using acc_t = f32x4;
    static constexpr int KS = 2;                                    // 16x16x128, 256 K per stage
    static constexpr int NACC = 4;
    static constexpr int kChunk2 = 0;
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 16; }
    static constexpr __device__ __host__ int frag_block(int lane, int ks) { return ks * 4 + lane / 16; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 4 + lane / 16; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (lane / 16) * 4 + r; }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 16; }
};
template <>
struct Mfma<32, kE2M1> {
    using acc_t = f32x16;
    static constexpr int KS = 4;                                    // 32x32x64, 256 K per stage
    static constexpr int NACC = 16;
    static constexpr int kChunk2 = 0;
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 32; }
    static constexpr __device__ __host__ int frag_block(int lane, int ks) { return ks * 2 + lane / 32; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 2 + lane / 32; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (r / 4) * 8 + (lane / 32) * 4 + (r % 4); }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 32; }
};

template <int MS, int FMT>
struct Frag {
    using t = bf16x8;
};
template <int MS>
struct Frag<MS, kE4M3> {
    using t = i32x8;
};
template <int MS>
struct Frag<MS, kE2M1> {
    using t = u32x4;
};

template <int MS, int FMT>
__device__ __forceinline__ typename Frag<MS, FMT>::t load_frag(const char* st, int off0, int off1) {
    if constexpr (FMT == kE4M3) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(st + off0);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(st + off1);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else if constexpr (FMT == kE2M1) {
        (void)off1;
        return *reinterpret_cast<const u32x4*>(st + off0);
    } else {
        (void)off1;
        return *reinterpret_cast<const bf16x8*>(st + off0);
    }
}

// SEL: block-scaled formats only, which byte of the scale registers sa / sb the instruction
// applies (op_sel)
template <int MS, int FMT, int SEL = 0>
__device__ __forceinline__ typename Mfma<MS, FMT>::acc_t mfma(typename Frag<MS, FMT>::t a, typename Frag<MS, FMT>::t b,
                                                              typename Mfma<MS, FMT>::acc_t c, int sa, int sb) {
    if constexpr (FMT == kBF16) {
        (void)sa;
        (void)sb;
        if constexpr (MS == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
        else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    } else if constexpr (FMT == kE4M3) {
        // format 0 = E4M3 for both operands; the scale byte SEL of each scale register
        if constexpr (MS == 32) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
        else return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
    } else {
        // format 4 = E2M1 for both operands, which take four registers each (the upper half of
        // the eight-register operand is not read)
        const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
        const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
        if constexpr (MS == 32) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SEL, sa, SEL, sb);
        else return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, SEL, sa, SEL, sb);
    }
}

template <int MS, int FMT>
__device__ __forceinline__ typename Mfma<MS, FMT>::acc_t acc_zero() {
    typename Mfma<MS, FMT>::acc_t z;
#pragma unroll
    for (int r = 0; r < Mfma<MS, FMT>::NACC; ++r) z[r] = 0.f;
    return z;
}

// ---------------------------------------------------------------------------------------
// fused output quantisation: the epilogue's bf16 tile (LDS, `pitch` bytes per row, rows
// [0, rows_valid) valid, BN_OUT columns from n0) quantised as the standalone quantisers would
// quantise the stored output: row-wise blocks of 32 columns (E4M3 codes or packed E2M1 codes,
// one scale byte each) and, for E4M3 with q_col, the group-aware column-wise blocks of 32 rows.
// A tile starts on a multiple of 128 rows of its group, so it owns whole column-wise blocks:
// the 4 (BM <= 128) or 8 (BM = 256) blocks from r_off / 32, those past the group's last row
// written as zeros (codes 0, scale 0), as the standalone pass writes them.
// ---------------------------------------------------------------------------------------
template <int BM, int BN_OUT>
__device__ __forceinline__ void quant_epilogue(const GemmParams& p, const char* lds, int pitch, int g, int r0,
                                               int r_off, int rows_valid, int n0, int tid, int col_end,
                                               int64_t ncols) {
    constexpr int RB = BN_OUT / 32;            // row-wise blocks per tile row
    const bool fp4 = p.q_fmt == kE2M1;
    for (int t = tid; t < BM * RB; t += kThreads) {
        const int row = t / RB, blk = t % RB;
        const int col = n0 + blk * 32;
        if (row >= rows_valid || col >= col_end) continue;   // col_end % 32 == 0: whole blocks only
        const char* src = lds + row * pitch + blk * 64;
        float v[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[c * 8 + 2 * i] = __uint_as_float(w[i] << 16);
                v[c * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int64_t r = (int64_t)(r0 + row);
        if (fp4) {
            const uint32_t byte = mx4_scale_byte(amax);
            const float inv = mx_inv_scale(byte);
            u32x4 out;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) word |= e2m1_code(v[w * 8 + i] * inv) << (4 * i);
                out[w] = word;
            }
            *reinterpret_cast<u32x4*>(p.q_row + r * p.ld_q_row + col / 2) = out;
            p.s_row[r * p.ld_s_row + col / 32] = (uint8_t)byte;
        } else {
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
            uint8_t* dst = p.q_row + r * p.ld_q_row + col;
            *reinterpret_cast<u32x4*>(dst) = out[0];
            *reinterpret_cast<u32x4*>(dst + 16) = out[1];
            p.s_row[r * p.ld_s_row + col / 32] = (uint8_t)byte;
        }
    }
    if (fp4 || p.q_col == nullptr) return;
    // column-wise: thread t takes block blk of the column pair cp (LDS reads of 4 bytes = two
    // columns); the 4 (8) threads of one column pair are adjacent lanes, so a column's 128
    // (256) code bytes go out as whole lines
    constexpr int NBT = BM <= 128 ? 4 : 8;     // column-wise blocks the tile owns
    const int bs0 = p.q_bs[g];
    const int nbg = p.q_bs[g + 1] - bs0;
    const int jb0 = r_off / 32;
    if (bs0 < 0 || nbg < jb0 + NBT || (int64_t)bs0 + nbg > p.q_col_blocks) return;   // never for consistent offsets
    const int64_t N = ncols;
    uint8_t* qg = p.q_col + 32 * N * bs0;
    uint8_t* sg = p.s_col + N * bs0;
    for (int t = tid; t < (BN_OUT / 2) * NBT; t += kThreads) {
        const int cp = t / NBT, blk = t % NBT;
        const int col = n0 + 2 * cp;
        if (col >= col_end) continue;             // col_end even: both columns or neither
        uint32_t pair[32];                         // rows' bf16 pairs (column col in the low half)
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int row = blk * 32 + i;
            pair[i] = row < rows_valid ? *reinterpret_cast<const uint32_t*>(lds + row * pitch + cp * 4) : 0u;
        }
        const int jb = jb0 + blk;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(half ? (pair[i] & 0xFFFF0000u) : (pair[i] << 16));
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
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
            const int64_t c = col + half;
            uint8_t* dst = qg + c * 32 * nbg + (int64_t)jb * 32;
            *reinterpret_cast<u32x4*>(dst) = out[0];
            *reinterpret_cast<u32x4*>(dst + 16) = out[1];
            sg[c * nbg + jb] = (uint8_t)byte;
        }
    }
}

// ---------------------------------------------------------------------------------------
// SwiGLU-backward epilogue (the data-gradient GEMM dh = dY W_down^T): the tile's dh values,
// already rounded to bf16 in LDS, meet the saved pre-activations g = aux[r, n] and
// u = aux[r, N + n]; dg and du (rounded to bf16, as moe_swiglu_backward stores them) replace
// dh in LDS and fill a second LDS tile, then go out as C = [dg | du] ([M, 2N], optional)
// and/or their quantised copies (2N columns), as the standalone SwiGLU backward followed by
// the quantisers would write them.
// ---------------------------------------------------------------------------------------
template <int BM>
__device__ __forceinline__ void swb_epilogue(const GemmParams& p, char* lds, int pitch, int g, int r0, int r_off,
                                             int rows_valid, int n0, int tid) {
    constexpr int BN = kBN;                    // dh columns of the tile
    constexpr int CH = BN / 8;                 // 16-byte chunks per tile row
    static_assert(2 * BM * (BN * 2 + 16) <= kMxData, "the dg and du tiles fit the operand stages");
    char* lds_u = lds + BM * pitch;            // the du tile (both fit the operand ring)
    // every g, u load of this thread goes out before the first is used (NB chunks per thread)
    constexpr int NB = cdiv(BM * CH, kThreads);
    u32x4 gv_all[NB], uv_all[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = tid + i * kThreads;
        const int row = c / CH, ch = c % CH;
        const int col = n0 + ch * 8;
        gv_all[i] = u32x4{0u, 0u, 0u, 0u};
        uv_all[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < BM * CH && row < rows_valid && col < p.N) {   // N % 8 == 0: a chunk is whole or absent
            const int64_t r = r0 + row;
            gv_all[i] = *reinterpret_cast<const u32x4*>(p.aux + (r * p.ld_aux + col) * 2);
            uv_all[i] = *reinterpret_cast<const u32x4*>(p.aux + (r * p.ld_aux + p.N + col) * 2);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = tid + i * kThreads;
        const int row = c / CH, ch = c % CH;
        const int col = n0 + ch * 8;
        if (c >= BM * CH || row >= rows_valid || col >= p.N) continue;
        const u32x4 hv = *reinterpret_cast<const u32x4*>(lds + row * pitch + ch * 16);
        const u32x4 gv = gv_all[i], uv = uv_all[i];
        u32x4 og, ou;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t pg = 0u, pu = 0u;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int sh = 16 * e;
                const float hh = __uint_as_float(((hv[w] >> sh) & 0xFFFFu) << 16);
                const float gg = __uint_as_float(((gv[w] >> sh) & 0xFFFFu) << 16);
                const float uu = __uint_as_float(((uv[w] >> sh) & 0xFFFFu) << 16);
                float dg, du;
                swiglu_grad(hh, gg, uu, dg, du);
                pg |= (uint32_t)f32_to_bf16(dg) << sh;
                pu |= (uint32_t)f32_to_bf16(du) << sh;
            }
            og[w] = pg;
            ou[w] = pu;
        }
        *reinterpret_cast<u32x4*>(lds + row * pitch + ch * 16) = og;
        *reinterpret_cast<u32x4*>(lds_u + row * pitch + ch * 16) = ou;
    }
    lds_barrier();
    if (!p.c_skip) {
        for (int c = tid; c < 2 * BM * CH; c += kThreads) {
            const int half = c / (BM * CH), cc = c % (BM * CH);
            const int row = cc / CH, ch = cc % CH;
            const int col = n0 + ch * 8;
            if (row >= rows_valid || col >= p.N) continue;
            const u32x4 v = *reinterpret_cast<const u32x4*>((half ? lds_u : lds) + row * pitch + ch * 16);
            *reinterpret_cast<u32x4*>(p.C + ((int64_t)(r0 + row) * p.ldc + half * p.N + col) * 2) = v;
        }
    }
    if (p.q_fmt != 0) {
        const int64_t ncols = 2 * (int64_t)p.N;
        quant_epilogue<BM, BN>(p, lds, pitch, g, r0, r_off, rows_valid, n0, tid, p.N, ncols);
        quant_epilogue<BM, BN>(p, lds_u, pitch, g, r0, r_off, rows_valid, p.N + n0, tid, 2 * p.N, ncols);
    }
}

// ---------------------------------------------------------------------------------------
// one output tile of BM rows x (256 B-rows) for group g
// ---------------------------------------------------------------------------------------
// Rows [r_off, r_off + BM) of group g's output (fewer at the group's end), columns of tile nt.
// RK (ragged K): every group computes the full M x N output over its own blocks
// offsets[g] .. offsets[g+1]-1 of 32 K elements, read from the group-major column-wise
// layout (group g's A block [M, 32 n_g] at A + 32 M offsets[g], row stride 32 n_g; likewise
// B with N rows and both scale blocks), and writes it at C + g * c_stride.
// PW: producer waves of the calling kernel (kPWaves in gemm_mfma_kernel; 0 in the 8-wave
// kernel that also runs 256-row tiles, whose MFMA waves issue their own loads)
template <int BM, bool SWIGLU, int FMT, bool RK, int PW = kPWaves>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, char* lds, int g, int r_off, int nt) {
    constexpr int LW = PW ? PW : kWaves;          // waves that issue the DMA loads
    constexpr int THR = (kWaves + PW) * kWave;    // threads of the workgroup
    constexpr bool MX = FMT != kBF16;                   // block-scaled operands (E8M0 scales)
    constexpr bool FP4 = FMT == kE2M1;
    constexpr int EB = MX ? 1 : 2;                      // operand element bytes (E2M1: half a byte)
    constexpr int KPS = FP4 ? 2 * kRowBytes : kRowBytes / EB;   // K elements per stage
    // wave grid WM x WN: 8 waves: 1x8 for 16 rows, else 2x4; 4 waves: 2x2 from 128 rows, else 1x4
    constexpr int WM = kWaves == 8 ? ((BM == 16) ? 1 : 2) : ((BM >= 128) ? 2 : 1);
    constexpr int WN = kWaves / WM;
    constexpr int MS = (BM / WM >= 32) ? 32 : 16;       // MFMA tile edge
    using MF = Mfma<MS, FMT>;
    using FragT = typename Frag<MS, FMT>::t;
    using ST = Stage<BM, FP4 ? kE2M1 : kE4M3>;
    constexpr int NKS = MF::KS;                          // MFMA k-steps per stage
    constexpr int ROWS_PER_INSTR = 1024 / kRowBytes;     // LDS rows filled by one 1 KiB DMA instruction
    constexpr int WTM = BM / WM;                         // rows per wave
    constexpr int WTN = kBN / WN;                        // B rows (tile columns) per wave
    constexpr int MI = WTM / MS;
    constexpr int NI = WTN / MS;
    constexpr int A_INSTR = BM / ROWS_PER_INSTR;         // 1 KiB DMA instructions for the A slice
    constexpr int A_PER_WAVE = cdiv(A_INSTR, LW);
    constexpr int B_PER_WAVE = kBN / ROWS_PER_INSTR / LW;
    constexpr int BN_OUT = SWIGLU ? kBN / 2 : kBN;
    constexpr int SDW = ST::kScaleDw;                    // scale dwords per row and stage
    constexpr int AS_GRP = cdiv(BM, 64);                 // 64-row groups of A (one scale instruction each)
    constexpr int BS_GRP = kBN / 64;
    constexpr int AS_INSTR = AS_GRP * SDW;               // scale dword instructions of a stage: A, then B
    constexpr int BS_INSTR = BS_GRP * SDW;
    // row tiles: scale batches (SPB stages each) in the two ring slots past the stages; piece q
    // of a batch brings 16 rows' 16 bytes (A rows for q < APC, then B rows)
    constexpr bool SCB = MX && !RK;
    constexpr int SPB = kScBatchBytes / (4 * SDW);        // stages per scale batch
    constexpr int APC = ST::kScaleRowsA / 16, NPC = APC + kBN / 16;
    constexpr int SC_PER_WAVE = !MX ? 0 : SCB ? cdiv(NPC, LW) : cdiv(AS_INSTR + BS_INSTR, LW);
    constexpr int NST = ST::kCount;
    constexpr int SB = SCB ? ST::kData : ST::kBytes;
    static_assert(!SCB || (NST * SB <= kMxData && SPB >= 2 && (ST::kScaleRowsA + kBN) * kScBatchBytes <= kScSlot),
                  "scale batch layout");
    static_assert(NST * SB <= pipe_bytes<FMT>(), "pipeline stages exceed the LDS ring");
    static_assert(NST <= 4, "the wait counts cover at most two later stages in flight");
    static_assert(BM < 256 || (BM * (kBN * 2 + 16) <= kPipeBytes), "bf16 epilogue tile must fit in LDS");
    static_assert(!SWIGLU || NI % 2 == 0, "SwiGLU needs gate and up fragments in every wave");
    static_assert(SC_PER_WAVE <= (SCB ? 6 : 3), "scale loads per wave");
    static_assert(!MX || PW == kPWaves, "block-scaled epilogues assume the persistent kernel's threads");

    if constexpr (BM == 256) {
        if (p.c_f32) return;   // never scheduled: 256-row tiles are only chosen for 2-byte outputs
    }
    // MXFP8: the lane index is made opaque per tile so its per-lane offsets are recomputed in
    // each tile (a few ALU operations) rather than hoisted out of the persistent tile loop and
    // kept live across it, which costs registers the MXFP8 tiles do not have (it spilled)
    int tid = threadIdx.x;
    if constexpr (MX) asm volatile("" : "+v"(tid));
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const bool producer = PW > 0 && wave >= kWaves;
    const int lw = PW ? wave - kWaves : wave;      // index among the load-issuing waves
    int row_begin, row_end;
    int nk = p.K / KPS;                                   // K slices
    char* Cg = p.C;
    // operand bases and row strides (bytes); scale bases and row strides (scale bytes)
    // row strides and offsets in bytes (E2M1: leading dimensions and strides counted in
    // elements, two per byte)
    auto bytes_of = [](int64_t elems) -> int64_t { return FP4 ? elems / 2 : elems * EB; };
    const char* a_base = p.A;
    int64_t a_ld = bytes_of(p.lda);
    const char* b_base = p.B + (RK ? 0 : bytes_of((int64_t)g * p.b_stride));
    int64_t b_ld = bytes_of(p.ldb);
    const uint8_t* as_base = p.a_scale;
    int64_t as_ld = p.lda_scale;
    const uint8_t* bs_base = p.b_scale ? p.b_scale + (RK ? 0 : (int64_t)g * p.b_scale_stride) : nullptr;
    int64_t bs_ld = p.ldb_scale;
    if constexpr (RK) {
        row_begin = 0;
        row_end = p.M;
        // clamp the block range into [0, K/32] and keep whole 128-element slices (both ends on
        // multiples of 4 blocks), so inconsistent offsets can never move a load outside A or B
        const int kb_max = p.K / 32;
        const int kb0 = min(max(p.offsets[g], 0), kb_max) & ~3;
        const int nbe = (max(min(p.offsets[g + 1], kb_max), kb0) - kb0) & ~3;   // blocks used
        nk = nbe / 4;
        a_base = p.A + (int64_t)32 * p.M * kb0;
        a_ld = (int64_t)32 * nbe;
        b_base = p.B + (int64_t)32 * p.N * kb0;
        b_ld = (int64_t)32 * nbe;
        as_base = p.a_scale + (int64_t)p.M * kb0;
        as_ld = nbe;
        bs_base = p.b_scale + (int64_t)p.N * kb0;
        bs_ld = nbe;
        Cg = p.C + (int64_t)g * p.c_stride * (p.c_f32 ? 4 : 2);
    } else if (p.uniform_rows > 0) {
        row_begin = min(g * p.uniform_rows, p.M);
        row_end = min(row_begin + p.uniform_rows, p.M);
        a_base = p.A + bytes_of((int64_t)g * p.a_group_stride);
    } else {
        group_rows(p.offsets, g, p.M, row_begin, row_end);
    }
    const int r0 = row_begin + r_off;                     // first C row of the tile
    const int n0 = nt * BN_OUT;                           // first output column

    auto a_row_of = [&](int row) -> int64_t {             // A row feeding tile row `row`
        const int r = min(r0 + row, row_end - 1);
        int64_t ar = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)(p.uniform_rows > 0 ? r - row_begin : r);
        return ar < 0 ? 0 : (ar >= p.A_rows ? p.A_rows - 1 : ar);
    };
    auto b_row_of = [&](int rho) -> int {                 // B row feeding LDS B-row `rho`
        if (SWIGLU) {
            // wave wn's WTN rows: first half gate rows, second half the matching up rows
            const int wnb = rho / WTN, within = rho % WTN;
            const int half = within / (WTN / 2), idx = within % (WTN / 2);
            return half * p.N + min(n0 + wnb * (WTN / 2) + idx, p.N - 1);
        }
        return min(n0 + rho, p.N - 1);
    };

    // per-lane global source pointers for the DMA loads (fixed for the whole K loop);
    // lane l of an instruction fills LDS row (instr * ROWS_PER_INSTR + l / kChunks)
    const char* a_src[A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
        const int instr = lw + LW * i;
        const int row = instr * ROWS_PER_INSTR + lane / kChunks;
        const int chunk = (lane % kChunks) ^ swz(row);
        a_src[i] = a_base + a_row_of(row) * a_ld + chunk * 16;
    }
#if MOE_BUF_DMA
    // buffer resources over the tile's operand bases; lane offsets stay below 2^32 for every
    // operand the host lets through (checked there), the scalar offset carries the K slice
#if MOE_DEBUG
    // the tile's operand extents (the last row needs only the K bytes); the K slice moves into
    // the range-checked lane offset below
    const int64_t kbytes = bytes_of(p.K);
    const int64_t a_rows_span = RK ? p.M : (p.uniform_rows > 0 ? p.uniform_rows : p.A_rows);
    const int64_t b_rows_span = RK ? p.N : (SWIGLU ? 2 * (int64_t)p.N : (int64_t)p.N);
    const int a_rec = (int)min<int64_t>((a_rows_span - 1) * a_ld + (RK ? a_ld : kbytes), 0xFFFFFFFFll);
    const int b_rec = (int)min<int64_t>((b_rows_span - 1) * b_ld + (RK ? b_ld : kbytes), 0xFFFFFFFFll);
#else
    const int a_rec = (int)0xFFFFFFFF, b_rec = (int)0xFFFFFFFF;
#endif
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, a_rec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, b_rec, 0x00020000);
    uint32_t a_voff[A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) a_voff[i] = (uint32_t)(a_src[i] - a_base);
#endif
    const char* b_src[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
        const int instr = lw * B_PER_WAVE + i;
        const int rho = instr * ROWS_PER_INSTR + lane / kChunks;
        const int chunk = (lane % kChunks) ^ swz(rho);
        b_src[i] = b_base + (int64_t)b_row_of(rho) * b_ld + chunk * 16;
    }
#if MOE_BUF_DMA
    uint32_t b_voff[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) b_voff[i] = (uint32_t)(b_src[i] - b_base);
#endif
    // MXFP8 scale rows: scale instruction q (0 .. AS_INSTR+BS_INSTR-1) is issued by load wave
    // q % LW as its (q / LW)-th scale load; instructions below AS_INSTR bring 64 A rows' scale
    // dwords, the others 64 B rows'
    // (row tiles: batch pieces, below, keep 32-bit row offsets from as_base / bs_base instead)
    const uint8_t* s_src[SC_PER_WAVE > 0 && !SCB ? SC_PER_WAVE : 1] = {};
    int s_lds[SC_PER_WAVE > 0 && !SCB ? SC_PER_WAVE : 1] = {};
    uint32_t s_off[SCB ? SC_PER_WAVE : 1] = {};
    if constexpr (SCB) {
        // batch pieces: lane l reads dword l % 4 of the batch in row 16 q + l / 4 (clamped to
        // the row's K range when the batch is issued) into slot byte 256 q + 4 l
#pragma unroll
        for (int u = 0; u < SC_PER_WAVE; ++u) {
            const int q = lw + LW * u;
            if (q < APC) s_off[u] = (uint32_t)(a_row_of(q * 16 + lane / 4) * as_ld);
            else if (q < NPC) s_off[u] = (uint32_t)((int64_t)b_row_of((q - APC) * 16 + lane / 4) * bs_ld);
        }
    } else if constexpr (MX) {
#pragma unroll
        for (int u = 0; u < SC_PER_WAVE; ++u) {
            const int q = lw + LW * u;
            if (q < AS_INSTR) {
                // dword h = q / AS_GRP of the stage's scales of rows 64 (q % AS_GRP) + lane
                const int h = q / AS_GRP, grp = q % AS_GRP;
                s_src[u] = as_base + a_row_of(grp * 64 + lane) * as_ld + 4 * h;
                s_lds[u] = ST::kScaleA + h * ST::kScaleRowsA * 4 + grp * 256;
            } else if (q < AS_INSTR + BS_INSTR) {
                const int h = (q - AS_INSTR) / BS_GRP, grp = (q - AS_INSTR) % BS_GRP;
                const int rho = grp * 64 + lane;
                s_src[u] = bs_base + (int64_t)b_row_of(rho) * bs_ld + 4 * h;
                s_lds[u] = ST::kScaleB + h * kBN * 4 + grp * 256;
            }
        }
    }

    // This wave's DMA loads of one stage, numbered 0 .. NLOADS-1: its A instructions, its B
    // instructions, then (MXFP8) its scale dword. issue_one(kt, l) issues load l of stage kt.
    constexpr int NLOADS = A_PER_WAVE + B_PER_WAVE + SC_PER_WAVE;
    auto issue_one = [&](int kt, auto l_tag) {
        constexpr int l = decltype(l_tag)::value;
        char* st = lds + (kt % NST) * SB;
        const int64_t koff = (int64_t)kt * kRowBytes;
        if constexpr (l < A_PER_WAVE) {
            const int instr = lw + LW * l;
#if MOE_BUF_DMA
            if (A_INSTR % LW == 0 || instr < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, MOE_LDS(st + instr * 1024), 16,
                                                         a_voff[l] + (MOE_DEBUG ? (uint32_t)koff : 0u),
                                                         MOE_DEBUG ? 0u : (uint32_t)koff, 0, 0);
#else
            if constexpr (A_INSTR % LW == 0) load_lds16(a_src[l] + koff, st + instr * 1024);
            else if (instr < A_INSTR) load_lds16(a_src[l] + koff, st + instr * 1024);
#endif
        } else if constexpr (l < A_PER_WAVE + B_PER_WAVE) {
            constexpr int i = l - A_PER_WAVE;
#if MOE_BUF_DMA
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, MOE_LDS(st + BM * kRowBytes + (lw * B_PER_WAVE + i) * 1024),
                                                     16, b_voff[i] + (MOE_DEBUG ? (uint32_t)koff : 0u),
                                                     MOE_DEBUG ? 0u : (uint32_t)koff, 0, 0);
#else
            load_lds16(b_src[i] + koff, st + BM * kRowBytes + (lw * B_PER_WAVE + i) * 1024);
#endif
        } else if constexpr (!SCB) {
            // 4 scale bytes (4 blocks of 32) per row and instruction; the stage's 4 * SDW blocks
            constexpr int u = l - A_PER_WAVE - B_PER_WAVE;
            if (lw + LW * u < AS_INSTR + BS_INSTR) load_lds4(s_src[u] + kt * 4 * SDW, st + s_lds[u]);
        }
    };
    // Scale batch b (stages b SPB .. b SPB + SPB - 1) goes out with the loads of stage
    // max(0, (b - 1) SPB + 2): the loads of a stage leave after barrier stage - 2, when the MFMA
    // waves are done with stage - 3 and so with batch b - 2, the slot's previous batch; and
    // before stage b SPB's own loads, so the waits for that stage cover it.
    auto issue_scales = [&](int kt) {
        if constexpr (SCB) {
            int b = -1;
            if (kt == 0) b = 0;
            else if ((kt + SPB - 2) % SPB == 0) b = (kt + SPB - 2) / SPB;
            if (b < 0 || b * SPB >= nk) return;
            char* slot = lds + kMxData + (b & 1) * kScSlot;
            const int dw = min(4 * b + lane % 4, nk * SDW - 1);   // the row's last dword at most
#pragma unroll
            for (int u = 0; u < SC_PER_WAVE; ++u) {
                const int q = lw + LW * u;
                if (q < NPC) load_lds4((q < APC ? as_base : bs_base) + s_off[u] + 4 * dw, slot + q * 256);
            }
        }
    };
    auto issue = [&](int kt) {
        issue_scales(kt);
        static_for<0>([&](auto l) { issue_one(kt, l); }, std::make_integer_sequence<int, NLOADS>{});
    };

    typename MF::acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = acc_zero<MS, FMT>();

    // Per-wave loads per stage differ (some waves issue no A or scale load); the wait count
    // uses the smallest, so every wave is sure its own loads of stage kt have landed.
    constexpr int LOADS_MIN = B_PER_WAVE + A_INSTR / LW;

    // per-lane LDS byte offsets of the first A and B fragment (fixed for the whole tile).
    // Fragment i (j) sits MS*i rows further down; MS is a multiple of 16 and swz() reads only
    // row bits 1..3, so its offset is the first one's plus the constant MS*i*kRowBytes, which
    // the LDS read takes as its immediate offset.
    static_assert(MS % 16 == 0, "fragment row steps must leave the swizzle unchanged");
    int a_off[NKS][2], b_off[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int chunk = MF::frag_chunk(lane, ks);
        const int ra = wm * WTM + MF::frag_row(lane);
        a_off[ks][0] = ra * kRowBytes + ((chunk ^ swz(ra)) << 4);
        a_off[ks][1] = ra * kRowBytes + (((chunk + MF::kChunk2) ^ swz(ra)) << 4);
        const int rb = wn * WTN + MF::frag_row(lane);
        b_off[ks][0] = BM * kRowBytes + rb * kRowBytes + ((chunk ^ swz(rb)) << 4);
        b_off[ks][1] = BM * kRowBytes + rb * kRowBytes + (((chunk + MF::kChunk2) ^ swz(rb)) << 4);
    }
    constexpr int FSTEP = MS * kRowBytes;   // bytes between consecutive fragments' rows
    constexpr bool DB_BF16 = FMT == kBF16;  // bf16 fragments are double-buffered in registers
    // compute(kt, kn): multiply stage kt; when kn >= 0 also issue this wave's loads of stage kn,
    // a share after the first MFMA of every k-step, so the DMA instructions queue while the
    // matrix core works instead of all waves issuing them back to back after the barrier.
    auto compute = [&](int kt, int kn) {
        const char* st = lds + (kt % NST) * SB;
        // block-scaled formats: this lane's rows' scale dwords of the stage, shifted so that byte
        // SEL of dword DW is the block of k-step ks for this lane (the instruction's op_sel picks it)
        int sa_w[MI][SDW], sb_w[NI][SDW];
        if constexpr (SCB) {
            const uint32_t sh0 = 8 * (MF::frag_block(lane, 0) - MF::frag_block(0, 0));
            const char* slot = lds + kMxData + ((kt / SPB) & 1) * kScSlot + 4 * SDW * (kt % SPB);
#pragma unroll
            for (int h = 0; h < SDW; ++h) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    sa_w[i][h] = (int)(*reinterpret_cast<const uint32_t*>(
                                           slot + 4 * h + (wm * WTM + i * MS + MF::frag_row(lane)) * kScBatchBytes) >> sh0);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    sb_w[j][h] = (int)(*reinterpret_cast<const uint32_t*>(
                                           slot + 4 * h + (ST::kScaleRowsA + wn * WTN + j * MS + MF::frag_row(lane)) *
                                                              kScBatchBytes) >> sh0);
            }
        } else if constexpr (MX) {
            const uint32_t sh0 = 8 * (MF::frag_block(lane, 0) - MF::frag_block(0, 0));
#pragma unroll
            for (int h = 0; h < SDW; ++h) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    sa_w[i][h] = (int)(*reinterpret_cast<const uint32_t*>(
                                           st + ST::kScaleA + h * ST::kScaleRowsA * 4 +
                                           (wm * WTM + i * MS + MF::frag_row(lane)) * 4) >> sh0);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    sb_w[j][h] = (int)(*reinterpret_cast<const uint32_t*>(
                                           st + ST::kScaleB + h * kBN * 4 + (wn * WTN + j * MS + MF::frag_row(lane)) * 4) >>
                                       sh0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < MI; ++i) sa_w[i][0] = 0;
#pragma unroll
            for (int j = 0; j < NI; ++j) sb_w[j][0] = 0;
        }
        // Fragments are double-buffered in registers (the LDS reads of k-step ks+1 go out before
        // the MFMAs of k-step ks); MOE_GEMM_MX_FRAG_DB=0 loads the MXFP8 fragments (twice the
        // size of bf16 ones) one k-step at a time instead
        constexpr bool DB = !MX || MOE_GEMM_MX_FRAG_DB;
        FragT af[DB ? 2 : 1][MI], bfr[DB ? 2 : 1][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = load_frag<MS, FMT>(st + i * FSTEP, a_off[0][0], a_off[0][1]);
#pragma unroll
        for (int j = 0; j < NI; ++j) bfr[0][j] = load_frag<MS, FMT>(st + j * FSTEP, b_off[0][0], b_off[0][1]);
        static_for<0>(
            [&](auto ks_tag) {
                constexpr int ks = decltype(ks_tag)::value;
                constexpr int cur = DB ? (ks & 1) : 0, nxt = DB ? (cur ^ 1) : 0;
                // the k-step's block of this lane: dword DW, byte SEL after the per-lane shift
                constexpr int DW = MX ? MF::frag_block(0, ks) / 4 : 0;
                constexpr int SEL = MX ? MF::frag_block(0, ks) % 4 : 0;
                static_assert(DW < SDW, "scale dword of the k-step");
                if constexpr (!DB && ks > 0) {
#pragma unroll
                    for (int i = 0; i < MI; ++i) af[0][i] = load_frag<MS, FMT>(st + i * FSTEP, a_off[ks][0], a_off[ks][1]);
#pragma unroll
                    for (int j = 0; j < NI; ++j) bfr[0][j] = load_frag<MS, FMT>(st + j * FSTEP, b_off[ks][0], b_off[ks][1]);
                }
                if constexpr (DB && ks + 1 < NKS) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        af[nxt][i] = load_frag<MS, FMT>(st + i * FSTEP, a_off[ks + 1][0], a_off[ks + 1][1]);
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        bfr[nxt][j] = load_frag<MS, FMT>(st + j * FSTEP, b_off[ks + 1][0], b_off[ks + 1][1]);
                }
                __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of the MFMAs below
                acc[0][0] = mfma<MS, FMT, SEL>(af[cur][0], bfr[cur][0], acc[0][0], sa_w[0][DW], sb_w[0][DW]);
                if (kn >= 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    static_for<0>(
                        [&](auto l) {
                            // k-step ks issues loads [ks*NLOADS/NKS, (ks+1)*NLOADS/NKS)
                            constexpr int lo = decltype(l)::value;
                            if constexpr (lo * NKS >= ks * NLOADS && lo * NKS < (ks + 1) * NLOADS) issue_one(kn, l);
                        },
                        std::make_integer_sequence<int, NLOADS>{});
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        if (i != 0 || j != 0)
                            acc[i][j] = mfma<MS, FMT, SEL>(af[cur][i], bfr[cur][j], acc[i][j], sa_w[i][DW], sb_w[j][DW]);
            },
            std::make_integer_sequence<int, NKS>{});
    };

    // Ring of NST LDS stages: stages kt+1 .. kt+NST-2 may still be streaming in when stage kt
    // is read, so each wave first waits until at most its own loads of those later stages are
    // pending (LOADS_MIN per stage); the barrier then makes every wave's loads of stage kt
    // visible and guarantees that the buffer refilled during compute(kt) (stage kt+NST-1,
    // last read in iteration kt-1) is no longer in use.
    if (nk > 0 && PW == 0) {    // only a ragged-K group with an empty range has no slice (C_g = 0)
        lds_barrier();   // the previous tile's epilogue may still read LDS
#pragma unroll
        for (int s0 = 0; s0 < NST - 1; ++s0)
            if (s0 < nk) issue(s0);
        for (int kt = 0; kt < nk; ++kt) {
            const int ahead = min(NST - 2, nk - 1 - kt);   // later stages possibly in flight
            if (ahead >= 2) wait_vm_lgkm0<2 * LOADS_MIN>();
            else if (ahead == 1) wait_vm_lgkm0<LOADS_MIN>();
            else wait_vm_lgkm0<0>();
            lds_barrier();
            compute(kt, kt + NST - 1 < nk ? kt + NST - 1 : -1);
        }
    } else if (nk > 0) {
        // producer waves issue every DMA load and wait for them; the MFMA waves only read LDS
        // and multiply. One barrier per stage: producers reach barrier kt with their loads of
        // stage kt landed; the buffer they refill after it (stage kt+NST-1) was last read by
        // compute(kt-1), which the MFMA waves finished before the same barrier.
        // bf16 (LATE): the MFMA waves cross barrier kt+1 before stage kt's last k-step, whose
        // fragments are already in registers, and read stage kt+1's first fragments under its
        // MFMAs, so no stage starts with the matrix core waiting on LDS reads. Barrier kt+1 then
        // follows every LDS read of stage kt, which is all the producers need before refilling
        // its slot; both roles pass nk + 1 barriers (the producers one more after their loop).
        constexpr bool LATE = FMT == kBF16 && !RK && DB_BF16;
        lds_barrier();
        if (producer) {   // two separate loops so that neither role keeps the other's registers live
#pragma unroll
            for (int s0 = 0; s0 < NST - 1; ++s0)
                if (s0 < nk) issue(s0);
            for (int kt = 0; kt < nk; ++kt) {
                const int ahead = min(NST - 2, nk - 1 - kt);
                if (ahead >= 2) wait_vm_lgkm0<2 * LOADS_MIN>();
                else if (ahead == 1) wait_vm_lgkm0<LOADS_MIN>();
                else wait_vm_lgkm0<0>();
                lds_barrier();
                if (kt + NST - 1 < nk) issue(kt + NST - 1);
            }
            if constexpr (LATE) lds_barrier();
        } else if constexpr (LATE) {
            static_assert(NKS >= 2 && (NKS - 1) % 2 == 1, "the last k-step uses fragment buffer 1");
            FragT fa[2][MI], fb[2][NI];
            auto rd = [&](int kt, int ks, int b) {
                const char* st = lds + (kt % NST) * SB;
#pragma unroll
                for (int i = 0; i < MI; ++i) fa[b][i] = load_frag<MS, FMT>(st + i * FSTEP, a_off[ks][0], a_off[ks][1]);
#pragma unroll
                for (int j = 0; j < NI; ++j) fb[b][j] = load_frag<MS, FMT>(st + j * FSTEP, b_off[ks][0], b_off[ks][1]);
            };
            auto mm = [&](int b) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j) acc[i][j] = mfma<MS, FMT, 0>(fa[b][i], fb[b][j], acc[i][j], 0, 0);
            };
            wait_vm_lgkm0<63>();
            lds_barrier();                       // barrier 0: stage 0 has landed
            rd(0, 0, 0);
            for (int kt = 0; kt < nk; ++kt) {
                static_for<0>(
                    [&](auto ks_tag) {
                        constexpr int ks = decltype(ks_tag)::value;
                        rd(kt, ks + 1, (ks + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of the MFMAs below
                        mm(ks & 1);
                    },
                    std::make_integer_sequence<int, NKS - 1>{});
                __builtin_amdgcn_sched_barrier(0);   // the k-step's MFMAs issue before the wait
                wait_vm_lgkm0<63>();             // this wave's LDS reads of stage kt are done
                lds_barrier();                   // barrier kt+1: stage kt+1 has landed
                rd(kt + 1, 0, 0);                // after the last stage: a stale slot, never used
                __builtin_amdgcn_sched_barrier(0);
                mm(1);
            }
        } else {
            for (int kt = 0; kt < nk; ++kt) {
                wait_vm_lgkm0<63>();   // this wave's LDS reads of compute(kt-1) are done
                lds_barrier();
                compute(kt, -1);
            }
        }
    }

    // ---- epilogue: values -> LDS (output dtype) -> 16-byte coalesced global stores ----
    wait_vm_lgkm0<0>();
    lds_barrier();
    const int esize = p.c_f32 ? 4 : 2;
    const int pitch = BN_OUT * esize + 16;
    const int rows_valid = min(BM, row_end - r0);
    constexpr int NO = SWIGLU ? NI / 2 : NI;       // output fragments per wave row block
    constexpr int WOUT = SWIGLU ? WTN / 2 : WTN;   // output columns per wave
    if (!producer)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int col = wn * WOUT + j * MS + MF::out_col(lane);
#pragma unroll
            for (int r = 0; r < MF::NACC; ++r) {
                const int row = wm * WTM + i * MS + MF::out_row(lane, r);
                float v;
                if (SWIGLU) {
                    const float gv = acc[i][j][r], uv = acc[i][j + NO][r];
                    v = silu(gv) * uv;
                    if (p.aux != nullptr && row < rows_valid && n0 + col < p.N) {
                        char* ap = p.aux + ((int64_t)(r0 + row) * p.ld_aux + n0 + col) * esize;
                        char* up = p.aux + ((int64_t)(r0 + row) * p.ld_aux + p.N + n0 + col) * esize;
                        if (p.c_f32) {
                            *reinterpret_cast<float*>(ap) = gv;
                            *reinterpret_cast<float*>(up) = uv;
                        } else {
                            *reinterpret_cast<uint16_t*>(ap) = f32_to_bf16(gv);
                            *reinterpret_cast<uint16_t*>(up) = f32_to_bf16(uv);
                        }
                    }
                } else {
                    v = acc[i][j][r];
                }
                char* dst = lds + row * pitch + col * esize;
                if (p.c_f32) *reinterpret_cast<float*>(dst) = v;
                else *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(v);
            }
        }
    lds_barrier();
    const int chunks_per_row = BN_OUT * esize / 16;
    const int cols_per_chunk = 16 / esize;
    // (block-scaled operand kernels only: the bf16 kernels' register budget has no room for it)
    if constexpr (!RK && MX && !SWIGLU) {
        if (p.swb) {
            swb_epilogue<BM>(p, lds, pitch, g, r0, r_off, rows_valid, n0, tid);
            return;
        }
    }
    if constexpr (!RK && MX) {
        if (p.q_fmt != 0) quant_epilogue<BM, BN_OUT>(p, lds, pitch, g, r0, r_off, rows_valid, n0, tid, p.N, p.N);
        if (p.c_skip) return;
    }
    for (int c = tid; c < BM * chunks_per_row; c += THR) {
        const int row = c / chunks_per_row, ch = c % chunks_per_row;
        const int col = n0 + ch * cols_per_chunk;
        if (row < rows_valid && col < p.N) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * pitch + ch * 16);
            u32x4* cp = reinterpret_cast<u32x4*>(Cg + ((int64_t)(r0 + row) * p.ldc + col) * esize);
            if (MOE_GEMM_C_NT == 2 || (MOE_GEMM_C_NT == 1 && !SWIGLU)) __builtin_nontemporal_store(v, cp);
            else *cp = v;
        }
    }
}

// Ordering of the tiles of one group: supertiles of SUP column tiles x all MT row tiles,
// row-major inside a supertile, so consecutive tiles share B panels and A panels.
template <int SUP = kSuper>
__device__ __forceinline__ void tile_coords(int L, int MT, int NT, int& mt, int& nt) {
    const int full = NT / SUP;
    if (L < full * MT * SUP) {
        const int s = L / (MT * SUP), rem = L % (MT * SUP);
        mt = rem / SUP;
        nt = s * SUP + rem % SUP;
    } else {
        const int rem = L - full * MT * SUP, w = NT - full * SUP;
        mt = rem / w;
        nt = full * SUP + rem % w;
    }
}



// ---------------------------------------------------------------------------------------
// Ragged-K (weight-gradient) tiles as one stream of K slices. A group averages a few K slices,
// so a tile that fills the ring from empty and then drains it through LDS spends most of
// its time waiting for memory. Here the load waves walk this workgroup's (tile, slice)
// sequence without stopping at tile boundaries (tiles of empty groups have no slice), ring
// slot = running slice count mod NST, one barrier per slice for both roles; the MFMA waves
// write each finished tile straight from registers through a wave-private 1 KiB LDS
// transpose (8 rows x 64 columns of bf16 at a time, one 128-byte line per 8 lanes), which
// lies outside the ring, so the next tile's first slices load during that epilogue. Both
// roles derive every tile's slice count the same way, so their barrier counts match.
// bf16 output only (the caller keeps fp32 outputs on the per-tile path).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void gemm_rk_stream(const GemmParams& p, char* lds, int slot) {
    constexpr int BM = 128, NST = Stage<BM>::kCount, SB = Stage<BM>::kBytes;
    constexpr int MS = 32, WM = 2, WN = kWaves / WM, WTM = BM / WM, WTN = kBN / WN;
    constexpr int MI = WTM / MS, NI = WTN / MS;
    using MF = Mfma<MS, kE4M3>;
    using FragT = typename Frag<MS, kE4M3>::t;
    constexpr int NKS = MF::KS;
    constexpr int ROWS_PER_INSTR = 1024 / kRowBytes, CH = kRowBytes / 16;
    constexpr int A_INSTR = BM / ROWS_PER_INSTR;
    constexpr int A_PER_WAVE = A_INSTR / kLWaves, B_PER_WAVE = kBN / ROWS_PER_INSTR / kLWaves;
    constexpr int AS_INSTR = BM / 64, BS_INSTR = kBN / 64;
    constexpr int SC_PER_WAVE = cdiv(AS_INSTR + BS_INSTR, kLWaves);
    constexpr int LOADS_MIN = A_PER_WAVE + B_PER_WAVE;
    static_assert(kPWaves > 0 && A_INSTR % kLWaves == 0 && MI >= 1 && NI >= 1, "load-wave layout");
    static_assert(kPipeBytes + kWaves * 1024 <= kLdsBytes, "epilogue staging fits past the ring");
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool producer = wave >= kWaves;
    const int per_group = p.MT * p.NT, total = p.G * per_group;
    const int kb_max = p.K / 32;
    // tile -> group, row/column tile and the group's whole 128-element K slices (as gemm_tile)
    auto tile_info = [&](int tile, int& g, int& mt, int& nt, int& kb0, int& nbe) {
        g = tile / per_group;
        if (p.NT >= kSuperRKMinNT) tile_coords<kSuperRK>(tile - g * per_group, p.MT, p.NT, mt, nt);
        else tile_coords(tile - g * per_group, p.MT, p.NT, mt, nt);
        kb0 = min(max(p.offsets[g], 0), kb_max) & ~3;
        nbe = (max(min(p.offsets[g + 1], kb_max), kb0) - kb0) & ~3;
    };
    lds_barrier();
    if (producer) {
#if MOE_BUF_DMA
        const int lw = wave - kWaves;
        int tile = slot, kt = 0, nk = 0, issued = 0;
        // placeholders until next_tile() finds a tile (no load is issued before it does)
        __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, 0, 0x00020000);
        __amdgpu_buffer_rsrc_t rsrc_b = rsrc_a;
        uint32_t a_voff[A_PER_WAVE], b_voff[B_PER_WAVE];
        const uint8_t* s_src[SC_PER_WAVE] = {};
        int s_lds[SC_PER_WAVE] = {};
        // from `tile` on, the next tile of this workgroup with a slice; sets its sources
        auto next_tile = [&]() -> bool {
            for (; tile < total; tile += gridDim.x) {
                int g, mt, nt, kb0, nbe;
                tile_info(tile, g, mt, nt, kb0, nbe);
                nk = nbe / 4;
                if (nk == 0) continue;
                const int r0 = mt * BM, n0 = nt * kBN;
                const int64_t ld = (int64_t)32 * nbe;
                const int a_rec = MOE_DEBUG ? (int)min<int64_t>((int64_t)p.M * ld, 0xFFFFFFFFll) : (int)0xFFFFFFFF;
                const int b_rec = MOE_DEBUG ? (int)min<int64_t>((int64_t)p.N * ld, 0xFFFFFFFFll) : (int)0xFFFFFFFF;
                rsrc_a = __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (int64_t)32 * p.M * kb0), (short)0, a_rec,
                                                           0x00020000);
                rsrc_b = __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (int64_t)32 * p.N * kb0), (short)0, b_rec,
                                                           0x00020000);
#pragma unroll
                for (int i = 0; i < A_PER_WAVE; ++i) {
                    const int row = (lw + kLWaves * i) * ROWS_PER_INSTR + lane / CH;
                    const int chunk = (lane % CH) ^ swz(row);
                    a_voff[i] = (uint32_t)(min(r0 + row, p.M - 1) * ld + chunk * 16);
                }
#pragma unroll
                for (int i = 0; i < B_PER_WAVE; ++i) {
                    const int rho = (lw * B_PER_WAVE + i) * ROWS_PER_INSTR + lane / CH;
                    const int chunk = (lane % CH) ^ swz(rho);
                    b_voff[i] = (uint32_t)(min(n0 + rho, p.N - 1) * ld + chunk * 16);
                }
#pragma unroll
                for (int u = 0; u < SC_PER_WAVE; ++u) {
                    const int q = lw + kLWaves * u;
                    if (q < AS_INSTR) {
                        s_src[u] = p.a_scale + (int64_t)p.M * kb0 + (int64_t)min(r0 + q * 64 + lane, p.M - 1) * nbe;
                        s_lds[u] = Stage<BM>::kScaleA + q * 256;
                    } else if (q < AS_INSTR + BS_INSTR) {
                        const int rho = (q - AS_INSTR) * 64 + lane;
                        s_src[u] = p.b_scale + (int64_t)p.N * kb0 + (int64_t)min(n0 + rho, p.N - 1) * nbe;
                        s_lds[u] = Stage<BM>::kScaleB + (q - AS_INSTR) * 256;
                    }
                }
                kt = 0;
                return true;
            }
            return false;
        };
        bool have = next_tile();
        // issue the next slice of the stream into ring slot issued % NST
        auto issue_next = [&]() {
            if (!have) return;
            char* st = lds + (issued % NST) * SB;
            const uint32_t koff = (uint32_t)(kt * kRowBytes);
#pragma unroll
            for (int i = 0; i < A_PER_WAVE; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, MOE_LDS(st + (lw + kLWaves * i) * 1024), 16,
                                                         a_voff[i] + (MOE_DEBUG ? koff : 0u), MOE_DEBUG ? 0u : koff, 0,
                                                         0);
#pragma unroll
            for (int i = 0; i < B_PER_WAVE; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b,
                                                         MOE_LDS(st + BM * kRowBytes + (lw * B_PER_WAVE + i) * 1024),
                                                         16, b_voff[i] + (MOE_DEBUG ? koff : 0u), MOE_DEBUG ? 0u : koff,
                                                         0, 0);
#pragma unroll
            for (int u = 0; u < SC_PER_WAVE; ++u)
                if (lw + kLWaves * u < AS_INSTR + BS_INSTR) load_lds4(s_src[u] + kt * 4, st + s_lds[u]);
            ++issued;
            if (++kt >= nk) {
                tile += gridDim.x;
                have = next_tile();
            }
        };
#pragma unroll
        for (int s0 = 0; s0 < NST - 1; ++s0) issue_next();
        for (int q = 0; q < issued; ++q) {
            static_assert(NST == 3, "one later slice in flight at each wait");
            if (q + 1 < issued) wait_vm_lgkm0<LOADS_MIN>();
            else wait_vm_lgkm0<0>();
            lds_barrier();
            issue_next();   // slice q + NST - 1 into the slot compute(q - 1) has left
        }
#endif
        return;
    }
    // ---- MFMA waves ----
    const int wm = wave / WN, wn = wave % WN;
    int a_off[NKS][2], b_off[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int chunk = MF::frag_chunk(lane, ks);
        const int ra = wm * WTM + MF::frag_row(lane), rb = wn * WTN + MF::frag_row(lane);
        a_off[ks][0] = ra * kRowBytes + ((chunk ^ swz(ra)) << 4);
        a_off[ks][1] = ra * kRowBytes + (((chunk + MF::kChunk2) ^ swz(ra)) << 4);
        b_off[ks][0] = BM * kRowBytes + rb * kRowBytes + ((chunk ^ swz(rb)) << 4);
        b_off[ks][1] = BM * kRowBytes + rb * kRowBytes + (((chunk + MF::kChunk2) ^ swz(rb)) << 4);
    }
    constexpr int FSTEP = MS * kRowBytes;
    char* stg = lds + kPipeBytes + wave * 1024;   // this wave's transpose buffer
    int q = 0;
    for (int tile = slot; tile < total; tile += gridDim.x) {
        int g, mt, nt, kb0, nbe;
        tile_info(tile, g, mt, nt, kb0, nbe);
        const int nk = nbe / 4;
        typename MF::acc_t acc[MI][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = acc_zero<MS, kE4M3>();
        for (int kt = 0; kt < nk; ++kt, ++q) {
            wait_vm_lgkm0<63>();   // this wave's LDS reads of the previous slice are done
            lds_barrier();
            const char* st = lds + (q % NST) * SB;
            int sa_w[MI], sb_w[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                sa_w[i] = *reinterpret_cast<const int*>(st + Stage<BM>::kScaleA + (wm * WTM + i * MS + MF::frag_row(lane)) * 4);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                sb_w[j] = *reinterpret_cast<const int*>(st + Stage<BM>::kScaleB + (wn * WTN + j * MS + MF::frag_row(lane)) * 4);
            FragT af[2][MI], bfr[2][NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) af[0][i] = load_frag<MS, kE4M3>(st + i * FSTEP, a_off[0][0], a_off[0][1]);
#pragma unroll
            for (int j = 0; j < NI; ++j) bfr[0][j] = load_frag<MS, kE4M3>(st + j * FSTEP, b_off[0][0], b_off[0][1]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int cur = ks & 1, nxt = cur ^ 1;
                if (ks + 1 < NKS) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        af[nxt][i] = load_frag<MS, kE4M3>(st + i * FSTEP, a_off[ks + 1][0], a_off[ks + 1][1]);
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        bfr[nxt][j] = load_frag<MS, kE4M3>(st + j * FSTEP, b_off[ks + 1][0], b_off[ks + 1][1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                const int sh = 8 * MF::frag_block(lane, ks);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = mfma<MS, kE4M3>(af[cur][i], bfr[cur][j], acc[i][j], (sa_w[i] >> sh) & 0xFF,
                                                   (sb_w[j] >> sh) & 0xFF);
            }
        }
        // epilogue: 8 output rows x 64 columns at a time through the wave's LDS buffer
        char* Cg = p.C + (int64_t)g * p.c_stride * 2;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q4 = 0; q4 < MS / 8; ++q4) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        *reinterpret_cast<uint16_t*>(stg + ((lane / 32) * 4 + rr) * 128 + (j * MS + lane % 32) * 2) =
                            f32_to_bf16(acc[i][j][4 * q4 + rr]);
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + (lane / 8) * 128 + (lane % 8) * 16);
                const int row = mt * BM + wm * WTM + i * MS + 8 * q4 + lane / 8;
                const int col = nt * kBN + wn * WTN + (lane % 8) * 8;
                if (row < p.M && col < p.N) {
                    u32x4* cp = reinterpret_cast<u32x4*>(Cg + ((int64_t)row * p.ldc + col) * 2);
                    if (MOE_GEMM_RK_C_NT) __builtin_nontemporal_store(v, cp);
                    else *cp = v;
                }
                asm volatile("" ::: "memory");
            }
    }
}

template <bool SWIGLU, int FMT, bool RK>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // XCD-aware slot: the hardware deals workgroups round-robin over the 8 XCDs, so give the
    // workgroups of one XCD consecutive slots (and hence consecutive tiles in each round)
    const int nxcd = (gridDim.x % 8 == 0) ? 8 : 1;
    const int per_xcd = gridDim.x / nxcd;
    const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
    if constexpr (RK) {
        if constexpr (MOE_GEMM_RK_STREAM && MOE_BUF_DMA && kPWaves > 0 && kWaves == 8) {
            if (!p.c_f32) {
                gemm_rk_stream(p, lds, slot);
                return;
            }
        }
        const int per_group = p.MT * p.NT;
        const int total = p.G * per_group;
        for (int tile = slot; tile < total; tile += gridDim.x) {
            const int g = tile / per_group;
            int mt, nt;
            if (p.NT >= kSuperRKMinNT) tile_coords<kSuperRK>(tile - g * per_group, p.MT, p.NT, mt, nt);
            else tile_coords(tile - g * per_group, p.MT, p.NT, mt, nt);
            gemm_tile<128, false, kE4M3, true>(p, lds, g, mt * 128, nt);
        }
        return;
    }
    // uniform groups: every group has the same rows, so the tile -> group map is fixed;
    // otherwise the schedule's tile prefix (position -> first tile) and order (position -> group)
    const bool uniform = p.uniform_rows > 0;
    const RowTiles rt_u = row_tiles(uniform ? p.uniform_rows : 0, false);
    const int per_group_u = rt_u.count() * p.NT;
    int32_t* ts = reinterpret_cast<int32_t*>(lds + pipe_bytes<FMT>());
    int total;
    if (uniform) {
        total = p.G * per_group_u;
    } else {
        for (int g = threadIdx.x; g <= p.G; g += kThreads) ts[g] = p.tile_start[g];
        __syncthreads();
        total = ts[p.G];
    }
    for (int tile = slot; tile < total; tile += gridDim.x) {
        int g, L;
        RowTiles rt;
        if (uniform) {
            g = tile / per_group_u;
            L = tile - g * per_group_u;
            rt = rt_u;
        } else {
            // schedule position = last q with ts[q] <= tile; its group from the order table
            int lo = 0, hi = p.G - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (ts[mid] <= tile) lo = mid;
                else hi = mid - 1;
            }
            g = min(max(p.order[lo], 0), p.G - 1);
            L = tile - ts[lo];
            int gb, ge;
            group_rows(p.offsets, g, p.M, gb, ge);
            rt = row_tiles(ge - gb, p.allow256 != 0);
        }
        int mt, nt, r_off, bm;
        tile_coords(L, rt.count(), p.NT, mt, nt);
        row_tile(rt, mt, r_off, bm);
        switch (bm) {
            case 16: gemm_tile<16, SWIGLU, FMT, false>(p, lds, g, r_off, nt); break;
            case 32: gemm_tile<32, SWIGLU, FMT, false>(p, lds, g, r_off, nt); break;
            case 64: gemm_tile<64, SWIGLU, FMT, false>(p, lds, g, r_off, nt); break;
            case 128: gemm_tile<128, SWIGLU, FMT, false>(p, lds, g, r_off, nt); break;
            default:
                // 256-row tiles are bf16 only (the fp8 fragments of a 256-row tile do not fit
                // the register budget next to its accumulators); never chosen for MXFP8
                if constexpr (FMT == kBF16 && MOE_GEMM_TILE256) gemm_tile<256, SWIGLU, FMT, false>(p, lds, g, r_off, nt);
                break;
        }
    }
}

// ---------------------------------------------------------------------------------------
// 256 x 256 tiles for the full 256-row chunks of bf16 groups (bf16 output, ragged rows, no
// G|U save), in gemm_split_kernel.
//
// A 128 x 256 tile asks L2 for 384 operand rows per 32,768 outputs, a 256 x 256 tile for 512
// rows per 65,536: a third fewer line requests per FLOP. Inside the persistent kernel (waves
// of 168 registers, two stages fed by the four load waves) 256-row tiles run slower; the
// shape measured faster on one MI355X is a workgroup of 8 waves, each a 64 x 128 wave tile
// (4 x 2), every wave issuing its own loads. Wave w brings 64 rows of a stage (A rows for
// w < 4, B rows otherwise) as whole 128-byte lines (64 bf16 of K) through buffer_load ... lds
// into a two-slot ring of 64 KiB stages; the loads of stage kt+2 leave right after the
// barrier that frees stage kt's slot, and that barrier sits before the stage's last k-step,
// so the next stage's first fragment reads hide under the MFMAs. Half-line (64-byte) K
// slices in deeper rings, four waves of 128 x 128 and operands staged through registers all
// measured slower. The K order and the MFMA (32x32x16 bf16, k-steps in ascending K within
// each 64-element stage) are the 128-row tiles', so a row's outputs are bit-identical
// whichever tile computes them.
// ---------------------------------------------------------------------------------------
constexpr int k256Threads = kWaves * kWave;                        // 8 waves, no producer waves
constexpr int k256Stage = 2 * 256 * kRowBytes;                      // 256 A rows, then 256 B rows
static_assert(kWaves == 8, "the 256-row tile's wave grid is 4 x 2 waves of 64 x 128");
static_assert(2 * k256Stage <= kPipeBytes && 256 * (kBN * 2 + 16) <= kPipeBytes, "256-row ring and staging fit");

// rows [r0, r0 + 256) of group g (rows [gb, ge)), column tile nt
template <bool SWIGLU>
__device__ __forceinline__ void gemm256_tile(const GemmParams& p, char* lds, int g, int ge, int r0, int nt) {
    constexpr int WN = 2, WTM = 64, WTN = 128, MI = 2, NI = 4, MS = 32;
    constexpr int BN_OUT = SWIGLU ? kBN / 2 : kBN;
    constexpr int NO = SWIGLU ? NI / 2 : NI;       // output fragments per wave row block
    constexpr int WOUT = SWIGLU ? WTN / 2 : WTN;   // output columns per wave
    constexpr int IPW = 64 / (1024 / kRowBytes);   // 1 KiB DMA instructions per wave and stage (64 rows)
    using MF = Mfma<MS, kBF16>;
    // the lane index is opaque per tile, so its per-lane offsets are derived here rather than
    // kept live across the persistent tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const bool loads_a = wave < 4;
    const int lrow0 = (wave % 4) * 64;             // first A (or B) row of this wave's loads
    const int nk = p.K / (kRowBytes / 2);
    const int64_t a_ld = p.lda * 2, b_ld = p.ldb * 2;
    const int n0 = nt * BN_OUT;
#if MOE_DEBUG
    // range-checked operand extents; the K slice moves into the checked lane offset
    const int64_t kbytes = (int64_t)p.K * 2;
    const int a_rec = (int)min<int64_t>((p.A_rows - 1) * a_ld + kbytes, 0xFFFFFFFFll);
    const int b_rec = (int)min<int64_t>(((SWIGLU ? 2 : 1) * (int64_t)p.N - 1) * b_ld + kbytes, 0xFFFFFFFFll);
#else
    const int a_rec = (int)0xFFFFFFFF, b_rec = (int)0xFFFFFFFF;
#endif
    // fragment offsets of a stage's four k-steps (as gemm_tile's)
    int a_off[4], b_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int chunk = MF::frag_chunk(lane, ks);
        const int ra = wm * WTM + MF::frag_row(lane), rb = 256 + wn * WTN + MF::frag_row(lane);
        a_off[ks] = ra * kRowBytes + ((chunk ^ swz(ra)) << 4);
        b_off[ks] = rb * kRowBytes + ((chunk ^ swz(rb)) << 4);
    }
    // this wave's DMA sources: lane l of instruction i fills LDS row lrow0 + 8 i + l / 8 of its
    // operand, slot l % 8, with global chunk (l % 8) ^ swz(row)
    const char* base = loads_a ? p.A : p.B + (int64_t)g * p.b_stride * 2;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, loads_a ? a_rec : b_rec, 0x00020000);
    uint32_t voff[IPW];
    if (loads_a) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int row = lrow0 + 8 * i + lane / 8;
            const int r = min(r0 + row, ge - 1);
            const int64_t ar = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
            const int64_t ac = ar < 0 ? 0 : (ar >= p.A_rows ? p.A_rows - 1 : ar);
            voff[i] = (uint32_t)(ac * a_ld + (((lane % 8) ^ swz(row)) << 4));
        }
    } else {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int row = lrow0 + 8 * i + lane / 8;
            int br;
            if (SWIGLU) {
                // wave wn's 128 B rows: 64 gate rows, then the matching 64 up rows
                const int wnb = row / WTN, within = row % WTN;
                br = (within / (WTN / 2)) * p.N + min(n0 + wnb * (WTN / 2) + within % (WTN / 2), p.N - 1);
            } else {
                br = min(n0 + row, p.N - 1);
            }
            voff[i] = (uint32_t)((int64_t)br * b_ld + (((lane % 8) ^ swz(row)) << 4));
        }
    }
    char* const dst0 = lds + (loads_a ? 0 : 256 * kRowBytes) + lrow0 * kRowBytes;
    auto issue = [&](int kt) {
        char* st = dst0 + (kt & 1) * k256Stage;
        const uint32_t koff = (uint32_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MOE_LDS(st + i * 1024), 16, voff[i] + (MOE_DEBUG ? koff : 0u),
                                                     MOE_DEBUG ? 0u : koff, 0, 0);
    };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = acc_zero<MS, kBF16>();
    bf16x8 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
    auto frags = [&](int kt, int ks, bf16x8 (&fa)[MI], bf16x8 (&fb)[NI]) {
        const char* st = lds + (kt & 1) * k256Stage;
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off[ks] + i * MS * kRowBytes);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(st + b_off[ks] + j * MS * kRowBytes);
    };
    auto mfmas = [&](const bf16x8 (&fa)[MI], const bf16x8 (&fb)[NI]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // one LDS fragment read after each of the first six MFMAs of a k-step
#define MOE_G256_ILV(grp)                                        \
    for (int q = 0; q < 6; ++q) {                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, grp);     \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, grp);     \
    }                                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, grp);
    lds_barrier();   // the previous tile's epilogue is done with LDS
    issue(0);
    if (nk > 1) {
        issue(1);
        wait_vm_lgkm0<IPW>();
    } else {
        wait_vm_lgkm0<0>();
    }
    lds_barrier();
    frags(0, 0, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
        frags(kt, 1, fa1, fb1);
        mfmas(fa0, fb0);
        MOE_G256_ILV(0)
        frags(kt, 2, fa0, fb0);
        mfmas(fa1, fb1);
        MOE_G256_ILV(1)
        frags(kt, 3, fa1, fb1);
        mfmas(fa0, fb0);
        MOE_G256_ILV(2)
        // own fragment reads of stage kt and own loads of stage kt+1 done; after the barrier
        // stage kt+1 is visible and nobody reads stage kt's slot, which stage kt+2 refills
        wait_vm_lgkm0<0>();
        lds_barrier();
        if (kt + 2 < nk) issue(kt + 2);
        frags(kt + 1, 0, fa0, fb0);   // after the last stage: a stale slot, never used
        mfmas(fa1, fb1);
        MOE_G256_ILV(3)
    }
#undef MOE_G256_ILV
    // ---- epilogue: values -> LDS (bf16) -> 16-byte coalesced stores ----
    wait_vm_lgkm0<0>();
    lds_barrier();
    constexpr int pitch = BN_OUT * 2 + 16;
    const int rows_valid = min(256, ge - r0);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int col = wn * WOUT + j * MS + MF::out_col(lane);
#pragma unroll
            for (int r = 0; r < MF::NACC; ++r) {
                const int row = wm * WTM + i * MS + MF::out_row(lane, r);
                const float v = SWIGLU ? silu(acc[i][j][r]) * acc[i][j + NO][r] : acc[i][j][r];
                *reinterpret_cast<uint16_t*>(lds + row * pitch + col * 2) = f32_to_bf16(v);
            }
        }
    lds_barrier();
    constexpr int chunks_per_row = BN_OUT * 2 / 16;
    for (int c = tid; c < 256 * chunks_per_row; c += k256Threads) {
        const int row = c / chunks_per_row, ch = c % chunks_per_row;
        const int col = n0 + ch * 8;
        if (row < rows_valid && col < p.N) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * pitch + ch * 16);
            u32x4* cp = reinterpret_cast<u32x4*>(p.C + ((int64_t)(r0 + row) * p.ldc + col) * 2);
            if (MOE_GEMM_C_NT == 2 || (MOE_GEMM_C_NT == 1 && !SWIGLU)) __builtin_nontemporal_store(v, cp);
            else *cp = v;
        }
    }
}

// bf16 ragged-row launches with the split: one persistent walk over the schedule, a group's
// first tiles being 256 x 256 over its full 256-row chunks and the rest the usual row tiles
// (their loads issued by the MFMA waves themselves: this workgroup has no producer waves).
template <bool SWIGLU>
__global__ __launch_bounds__(k256Threads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_split_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int nxcd = (gridDim.x % 8 == 0) ? 8 : 1;   // XCD-aware slots, as gemm_mfma_kernel
    const int per_xcd = gridDim.x / nxcd;
    const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
    int32_t* ts = reinterpret_cast<int32_t*>(lds + kPipeBytes);
    for (int g = threadIdx.x; g <= p.G; g += k256Threads) ts[g] = p.tile_start[g];
    __syncthreads();
    const int total = ts[p.G];
    for (int tile = slot; tile < total; tile += gridDim.x) {
        int lo = 0, hi = p.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ts[mid] <= tile) lo = mid;
            else hi = mid - 1;
        }
        const int g = min(max(p.order[lo], 0), p.G - 1);
        const int L = tile - ts[lo];
        int gb, ge;
        group_rows(p.offsets, g, p.M, gb, ge);
        const int c256 = chunk256_rows(ge - gb, p.split256);
        const int t256 = (c256 / 256) * p.NT;
        int mt, nt;
        if (L < t256) {
            tile_coords(L, c256 / 256, p.NT, mt, nt);
            gemm256_tile<SWIGLU>(p, lds, g, ge, gb + 256 * mt, nt);
            continue;
        }
        const RowTiles rt = row_tiles(ge - gb - c256, false);
        int r_off, bm;
        tile_coords(L - t256, rt.count(), p.NT, mt, nt);
        row_tile(rt, mt, r_off, bm);
        r_off += c256;
        switch (bm) {
            case 16: gemm_tile<16, SWIGLU, kBF16, false, 0>(p, lds, g, r_off, nt); break;
            case 32: gemm_tile<32, SWIGLU, kBF16, false, 0>(p, lds, g, r_off, nt); break;
            case 64: gemm_tile<64, SWIGLU, kBF16, false, 0>(p, lds, g, r_off, nt); break;
            default: gemm_tile<128, SWIGLU, kBF16, false, 0>(p, lds, g, r_off, nt); break;
        }
    }
}

// ---------------------------------------------------------------------------------------
// fp32 grouped GEMM: one thread per output element, sequential fp32 dot products.
// Meant for small fp32 layers (correctness, not speed).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p, int64_t M, int swiglu) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * p.N) return;
    const int r = (int)(idx / p.N), n = (int)(idx % p.N);
    int g = -1;
    for (int q = 0; q < p.G; ++q) {     // small G only: a linear search is fine
        int b, e;
        group_rows(p.offsets, q, p.M, b, e);
        if (r >= b && r < e) { g = q; break; }
    }
    if (g < 0) return;
    int64_t ar = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
    ar = ar < 0 ? 0 : (ar >= p.A_rows ? p.A_rows - 1 : ar);
    const float* a = reinterpret_cast<const float*>(p.A) + ar * p.lda;
    const float* b = reinterpret_cast<const float*>(p.B) + (int64_t)g * p.b_stride;
    float s = 0.f, u = 0.f;
    for (int kk = 0; kk < p.K; ++kk) s = fmaf(a[kk], b[(int64_t)n * p.ldb + kk], s);
    float v = s;
    if (swiglu) {
        for (int kk = 0; kk < p.K; ++kk) u = fmaf(a[kk], b[(int64_t)(p.N + n) * p.ldb + kk], u);
        v = silu(s) * u;
        if (p.aux) {
            float* ax = reinterpret_cast<float*>(p.aux);
            ax[(int64_t)r * p.ld_aux + n] = s;
            ax[(int64_t)r * p.ld_aux + p.N + n] = u;
        }
    }
    if (p.c_f32) reinterpret_cast<float*>(p.C)[(int64_t)r * p.ldc + n] = v;
    else reinterpret_cast<uint16_t*>(p.C)[(int64_t)r * p.ldc + n] = f32_to_bf16(v);
}

int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <bool SWIGLU, int FMT, bool RK>
bool set_lds_attr() {
    static bool done = false;
    if (!done) {
        if (hipFuncSetAttribute((const void*)gemm_mfma_kernel<SWIGLU, FMT, RK>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes<FMT>()) != hipSuccess)
            return false;
        done = true;
    }
    return true;
}

template <bool SWIGLU>
moe_status_t launch_split(const GemmParams& p, int grid, hipStream_t s) {
    static bool attr = false;
    if (!attr) {
        if (hipFuncSetAttribute((const void*)gemm_split_kernel<SWIGLU>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsBytes) != hipSuccess)
            return MOE_EHIP;
        attr = true;
    }
    hipLaunchKernelGGL((gemm_split_kernel<SWIGLU>), dim3((unsigned)grid), dim3(k256Threads), kLdsBytes, s, p);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

template <bool SWIGLU, int FMT, bool RK = false>
moe_status_t launch(const GemmParams& p, int grid, hipStream_t s) {
    if (!set_lds_attr<SWIGLU, FMT, RK>()) return MOE_EHIP;
    hipLaunchKernelGGL((gemm_mfma_kernel<SWIGLU, FMT, RK>), dim3((unsigned)grid), dim3(kThreads), lds_bytes<FMT>(), s,
                       p);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace
}  // namespace moe

size_t moe_gemm_workspace_bytes(int32_t G) {
    if (G < 1) G = 1;
    return ((2 * (size_t)G + 1) * 4 + 255) & ~size_t(255);   // tile_start [G+1], order [G]
}

static inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

extern "C" moe_status_t moe_grouped_gemm(const moe_gemm_args_t* a, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    if (!a) return MOE_EINVAL;
    if (a->G < 1 || a->G > moe::kMaxGroups || !a->offsets) return MOE_EINVAL;
    if (a->M < 0 || a->N <= 0 || a->K <= 0 || a->N % 8 != 0 || a->N > (1 << 24) || a->K > (1 << 24))
        return MOE_EINVAL;
    if (a->M > INT32_MAX / 2) return MOE_EINVAL;
    if (a->epilogue != MOE_EPI_NONE && a->epilogue != MOE_EPI_SWIGLU && a->epilogue != MOE_EPI_SWIGLU_BWD)
        return MOE_EINVAL;
    const bool swb = a->epilogue == MOE_EPI_SWIGLU_BWD;
    if (swb) {
        // block-scaled operands, ragged rows, bf16 output; the saved pre-activations are read
        if ((a->a_dtype != MOE_E4M3 && a->a_dtype != MOE_E2M1) || a->ragged_k || a->c_dtype != MOE_BF16)
            return MOE_ENOTSUP;
        if (!a->aux || a->ld_aux < 2 * a->N || a->ld_aux % 8 || !moe_aligned16(a->aux)) return MOE_EINVAL;
        if (a->N > INT32_MAX / 2 || (a->C && a->ldc < 2 * a->N)) return MOE_EINVAL;
    }
    if (a->a_dtype != a->b_dtype) return MOE_ENOTSUP;
    if (a->a_dtype != MOE_BF16 && a->a_dtype != MOE_F32 && a->a_dtype != MOE_E4M3 && a->a_dtype != MOE_E2M1)
        return MOE_ENOTSUP;
    // block-scaled row tiles: the scale ring leaves LDS for the schedule of 1023 groups
    if (a->a_dtype == MOE_E2M1 && a->ragged_k) return MOE_ENOTSUP;
    if ((a->a_dtype == MOE_E4M3 || a->a_dtype == MOE_E2M1) && !a->ragged_k && a->G > moe::max_groups<moe::kE4M3>())
        return MOE_ENOTSUP;
    if (a->c_dtype != MOE_BF16 && a->c_dtype != MOE_F32) return MOE_ENOTSUP;
    if (a->a_dtype == MOE_F32 && a->c_dtype != MOE_F32) return MOE_ENOTSUP;
    if (a->ragged_k != 0 && a->ragged_k != 1) return MOE_EINVAL;
    if (a->ragged_k) {
        // weight-gradient form: MXFP8 only, plain epilogue, A is [M, K] and B is [N, K]
        if (a->a_dtype != MOE_E4M3 || a->epilogue != MOE_EPI_NONE) return MOE_ENOTSUP;
        if (a->a_rows || a->aux || a->b_group_stride != 0 || a->b_scale_group_stride != 0) return MOE_EINVAL;
        if (a->A_rows != a->M || a->c_group_stride < a->M * a->ldc) return MOE_EINVAL;
        // the operands are the column-wise quantiser's group-major blocks: the leading
        // dimensions state the capacity, [M, K] and [N, K] codes, [M, K/32] and [N, K/32] scales
        if (a->lda != a->K || a->ldb != a->K || a->lda_scale != a->K / 32 || a->ldb_scale != a->K / 32)
            return MOE_EINVAL;
    }
    // fused output quantisation: ragged rows, bf16 output, whole 32-column blocks
    const bool quant = a->q_dtype != 0;
    if (quant) {
        if (a->q_dtype != MOE_E4M3 && a->q_dtype != MOE_E2M1) return MOE_ENOTSUP;
        if (a->ragged_k || a->c_dtype != MOE_BF16 || (a->a_dtype != MOE_E4M3 && a->a_dtype != MOE_E2M1))
            return MOE_ENOTSUP;
        if (a->q_col && a->q_dtype != MOE_E4M3) return MOE_ENOTSUP;
        if (a->N % 32 != 0) return MOE_EINVAL;
    } else if (a->q_row || a->s_row || a->q_col || a->s_col || a->q_block_start) {
        return MOE_EINVAL;
    }
    if (a->M == 0) return MOE_OK;
    if (!a->A || !a->B || (!a->C && !quant) || a->A_rows <= 0) return MOE_EINVAL;
    if (quant) {
        const int64_t qn = swb ? 2 * a->N : a->N;   // columns of the quantised matrix
        const int64_t row_bytes = a->q_dtype == MOE_E2M1 ? qn / 2 : qn;
        if (!a->q_row || !a->s_row || !moe_aligned16(a->q_row) || a->ld_q_row < row_bytes || a->ld_q_row % 16 ||
            a->ld_s_row < qn / 32)
            return MOE_EINVAL;
        if (a->q_col) {
            // capacity for every group's blocks, whatever the device offsets hold (as
            // moe_group_quant_mxfp8's column-wise mode: 4 (ceil(M / 128) + G) blocks)
            const int64_t need = 4 * (moe::cdiv<int64_t>(a->M, 128) + a->G);
            if (!a->s_col || !a->q_block_start || !moe_aligned16(a->q_col) || a->q_col_blocks < need)
                return MOE_EINVAL;
        } else if (a->s_col || a->q_block_start) {
            return MOE_EINVAL;
        }
    }
    // groups' B matrices are only read, so they may overlap (e.g. K slices of one matrix)
    if (a->lda < a->K || a->ldb < a->K || (a->C && a->ldc < (swb ? 2 : 1) * a->N) || a->b_group_stride < 0)
        return MOE_EINVAL;
    if (a->aux && (a->epilogue == MOE_EPI_NONE || a->ld_aux < 2 * a->N)) return MOE_EINVAL;
    if (!workspace || workspace_bytes < moe_gemm_workspace_bytes(a->G)) return MOE_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const bool fp4 = a->a_dtype == MOE_E2M1;
    const bool mx = a->a_dtype == MOE_E4M3 || fp4;

    moe::GemmParams p{};
    p.offsets = a->offsets;
    p.G = a->G;
    p.M = (int)a->M;
    p.N = (int)a->N;
    p.K = (int)a->K;
    p.A = (const char*)a->A;
    p.lda = a->lda;
    p.A_rows = a->A_rows;
    p.a_rows = a->a_rows;
    p.B = (const char*)a->B;
    p.ldb = a->ldb;
    p.b_stride = a->b_group_stride;
    p.C = (char*)a->C;
    p.ldc = a->ldc;
    p.c_f32 = a->c_dtype == MOE_F32 ? 1 : 0;
    p.aux = (char*)a->aux;
    p.ld_aux = a->ld_aux;
    p.a_scale = a->a_scale;
    p.lda_scale = a->lda_scale;
    p.b_scale = a->b_scale;
    p.ldb_scale = a->ldb_scale;
    p.b_scale_stride = a->b_scale_group_stride;
    p.tile_start = (const int32_t*)workspace;
    p.order = (const int32_t*)workspace + (a->G + 1);
    p.c_stride = a->c_group_stride;
    p.allow256 = (MOE_GEMM_TILE256 && a->c_dtype != MOE_F32 && a->a_dtype == MOE_BF16) ? 1 : 0;
    p.q_fmt = !quant ? 0 : a->q_dtype == MOE_E2M1 ? moe::kE2M1 : moe::kE4M3;
    p.q_row = a->q_row;
    p.ld_q_row = a->ld_q_row;
    p.s_row = a->s_row;
    p.ld_s_row = a->ld_s_row;
    p.q_col = a->q_col;
    p.s_col = a->s_col;
    p.q_bs = a->q_block_start;
    p.q_col_blocks = a->q_col_blocks;
    p.c_skip = a->C == nullptr ? 1 : 0;
    p.swb = swb ? 1 : 0;
    const bool swiglu = a->epilogue == MOE_EPI_SWIGLU;
    // bf16 operands and output, ragged rows, A read in row order, plain or SwiGLU epilogue
    // without the G|U save: gemm_split_kernel, full 256-row chunks of large groups as 256 x 256
    // tiles (none while M < 256)
    const bool split = MOE_GEMM_SPLIT256 && a->a_dtype == MOE_BF16 && a->c_dtype == MOE_BF16 && !a->ragged_k &&
                       !quant && !swb && !a->aux && !a->a_rows && p.allow256 == 0 && a->M >= 256;
    p.split256 = !split ? 0 : a->K >= MOE_GEMM_SPLIT_LONGK ? std::max(MOE_GEMM_SPLIT_MIN_ROWS_LONGK, 256)
                                                            : std::max(MOE_GEMM_SPLIT_MIN_ROWS, 256);

#if MOE_DEBUG
    {
        // the device index data, validated on the host: offsets non-decreasing within [0, M]
        // (ragged K: [0, K/32] on multiples of 4 blocks), gather indices within [0, A_rows)
        std::vector<int32_t> off, ar;
        if (!moe_debug_fetch_i32(a->offsets, a->G + 1, s, off)) return MOE_EHIP;
        const int64_t lim = a->ragged_k ? a->K / 32 : a->M;
        for (int g = 0; g <= a->G; ++g)
            if (off[g] < 0 || off[g] > lim || (g > 0 && off[g] < off[g - 1]) || (a->ragged_k && off[g] % 4))
                return MOE_EINVAL;
        if (a->a_rows) {
            if (!moe_debug_fetch_i32(a->a_rows, a->M, s, ar)) return MOE_EHIP;
            for (int64_t r = off[0]; r < off[a->G]; ++r)
                if (ar[r] < 0 || ar[r] >= a->A_rows) return MOE_EINVAL;
        }
    }
#endif
    if (a->a_dtype == MOE_F32) {
        p.NT = 0;
        const int64_t n = a->M * a->N;
        hipLaunchKernelGGL(moe::gemm_f32_kernel, dim3((unsigned)moe::cdiv<int64_t>(n, 256)), dim3(256), 0, s, p,
                           a->M, swiglu ? 1 : 0);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // MFMA paths: 128-byte K slices (64 bf16, 128 E4M3 or 256 E2M1 values); sizes in bytes
    // (E2M1 packs two values per byte, so its element counts must be even)
    const int64_t eb2 = fp4 ? 1 : mx ? 2 : 4;   // bytes per two elements
    auto bytes = [eb2](int64_t elems) { return elems * eb2 / 2; };
    if (fp4 && (a->lda % 2 || a->ldb % 2 || a->b_group_stride % 2)) return MOE_EINVAL;
    if (a->K % (2 * moe::kRowBytes / eb2) != 0) return MOE_EINVAL;
    if (!moe_aligned16(a->A) || !moe_aligned16(a->B) || (a->C && !moe_aligned16(a->C))) return MOE_EINVAL;
    if (bytes(a->lda) % 16 || bytes(a->ldb) % 16 || a->ldc % 8 || bytes(a->b_group_stride) % 16) return MOE_EINVAL;
    if (a->aux && (!moe_aligned16(a->aux) || a->ld_aux % 8)) return MOE_EINVAL;
    if (mx) {
        if (!a->a_scale || !a->b_scale || !aligned4(a->a_scale) || !aligned4(a->b_scale)) return MOE_EINVAL;
        // row tiles address scale rows by 32-bit offsets from the scale bases
        if (!a->ragged_k && (a->A_rows * a->lda_scale >= ((int64_t)1 << 32) ||
                             (swiglu ? 2 : 1) * a->N * a->ldb_scale >= ((int64_t)1 << 32)))
            return MOE_ENOTSUP;
        if (a->lda_scale < a->K / 32 || a->ldb_scale < a->K / 32 || a->lda_scale % 4 || a->ldb_scale % 4 ||
            a->b_scale_group_stride < 0 || a->b_scale_group_stride % 4)
            return MOE_EINVAL;
    }
    const int bn_out = swiglu ? moe::kBN / 2 : moe::kBN;
    p.NT = (int)moe::cdiv<int64_t>(a->N, bn_out);
    if (MOE_GEMM_BUFFER_LDS) {
        // buffer DMA adds 32-bit lane offsets to each tile's operand base: every operand region
        // a tile addresses (plus the K extent) must stay below 4 GiB
        const int64_t lim = (int64_t)1 << 32;
        const int64_t kb = bytes(a->K);
        const int64_t a_span = a->ragged_k ? a->M * kb : a->A_rows * bytes(a->lda);
        const int64_t b_span = a->ragged_k ? a->N * kb : (swiglu ? 2 : 1) * a->N * bytes(a->ldb);
        if (a_span + kb >= lim || b_span + kb >= lim) return MOE_ENOTSUP;
    }
    if (a->ragged_k) {
        // every group: MT x NT tiles of 128 x 256 over its own K range; no schedule needed
        if (a->ldc % 8 || (a->c_group_stride % 8)) return MOE_EINVAL;
        p.MT = (int)moe::cdiv<int64_t>(a->M, 128);
        const int64_t tiles = (int64_t)p.MT * p.NT * a->G;
        if (tiles > INT32_MAX) return MOE_EINVAL;
        const int grid = (int)std::min<int64_t>((int64_t)moe::num_cus(), tiles);
        return moe::launch<false, moe::kE4M3, true>(p, grid, s);
    }
    hipLaunchKernelGGL(moe::gemm_schedule_kernel, dim3(1), dim3(1024), 0, s, a->offsets, a->G, p.M, p.NT,
                       p.allow256, (int32_t*)workspace, (int32_t*)workspace + (a->G + 1),
                       a->q_col ? a->q_block_start : nullptr, p.split256);
    MOE_CHECK_LAUNCH();
    // enough persistent workgroups to fill every CU, never more than the tile bound
    const int64_t bound = (a->M / 16 + a->G) * (int64_t)p.NT;
    const int grid = (int)std::min<int64_t>((int64_t)moe::num_cus(), std::max<int64_t>(bound, 1));
    if (split) return swiglu ? moe::launch_split<true>(p, grid, s) : moe::launch_split<false>(p, grid, s);
    if (swiglu)
        return fp4 ? moe::launch<true, moe::kE2M1>(p, grid, s)
                   : mx ? moe::launch<true, moe::kE4M3>(p, grid, s) : moe::launch<true, moe::kBF16>(p, grid, s);
    return fp4 ? moe::launch<false, moe::kE2M1>(p, grid, s)
               : mx ? moe::launch<false, moe::kE4M3>(p, grid, s) : moe::launch<false, moe::kBF16>(p, grid, s);
}

// Internal entry (route.hip): a bf16 K-split projection as one launch over KS uniform groups,
// C[s T + t, n] = sum over k in slice s of x[t, k] w[n, k], fp32 out (the slices' partial sums).
// Group s reads columns [s K, (s+1) K) of x and of w in place (K = d / KS): no row index,
// offsets or schedule kernel are needed. Arguments as moe_grouped_gemm's checks require.
moe_status_t moe_gemm_ksplit_f32(const void* x, const void* w, int64_t T, int64_t d, int32_t N, int32_t KS, float* C,
                                 hipStream_t s) {
    if (!x || !w || !C || T <= 0 || d <= 0 || N <= 0 || KS < 1) return MOE_EINVAL;
    if (N % 8 != 0 || d % (64 * (int64_t)KS) != 0 || T * KS > INT32_MAX / 2 || N > (1 << 24)) return MOE_EINVAL;
    if (!moe_aligned16(x) || !moe_aligned16(w) || !moe_aligned16(C)) return MOE_EINVAL;
    const int64_t lim = (int64_t)1 << 32;   // buffer DMA: 32-bit lane offsets from each group's base
    if (T * d * 2 >= lim || (int64_t)N * d * 2 >= lim) return MOE_ENOTSUP;
    moe::GemmParams p{};
    p.G = KS;
    p.M = (int)(T * KS);
    p.N = N;
    p.K = (int)(d / KS);
    p.NT = (int)moe::cdiv<int64_t>(N, moe::kBN);
    p.A = (const char*)x;
    p.lda = d;
    p.A_rows = T;
    p.B = (const char*)w;
    p.ldb = d;
    p.b_stride = d / KS;
    p.C = (char*)C;
    p.ldc = N;
    p.c_f32 = 1;
    p.uniform_rows = (int)T;
    p.a_group_stride = d / KS;
    const int64_t row_tiles = T <= 128 ? 1 : T / 128 + (T % 128 ? 1 : 0);
    const int64_t tiles = row_tiles * p.NT * KS;
    const int grid = (int)std::min<int64_t>((int64_t)moe::num_cus(), tiles);
    return moe::launch<false, moe::kBF16>(p, grid, s);
}

// moe_grouped_gemm: one launch computes every group's product at its real row count.
//
// [Blog] "Optimisation 1": a grouped GEMM runs all experts' matmuls in one kernel call, each
// at its actual token count, and computes only the regions that hold real tokens; the
// alternatives (a host loop over experts after a device-to-host copy of the counts, or a
// batched GEMM padded to the worst case) are what it replaces. [Blog] Figure 3 paragraph:
// the grouped MLP is two such GEMMs, gate/up then down.
//
// Design (gfx950):
//  * A one-workgroup schedule kernel turns the device-resident group offsets into a tile
//    prefix (tiles of group g start at tile_start[g]); the host never sees group sizes.
//  * Each group gets its own tile height BM in {16, 32, 64, 128} from its row count, so tiny
//    groups do not pay for 128-row tiles and empty groups get no tile at all.
//  * Persistent workgroups (one per CU, 4 waves) walk the tile list; tiles are ordered
//    group by group, in supertiles of 4 column tiles x all row tiles, and handed out so the
//    32 CUs of one XCD work on 32 consecutive tiles (shared A/B panels hit that XCD's L2).
//  * Operands go global -> LDS with 16-byte DMA loads (no VGPR staging) through a 3-stage
//    ring of 64-wide K slices; LDS rows are XOR-swizzled so the MFMA fragment reads are
//    bank-conflict free; products use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//  * The epilogue (optional SwiGLU) goes through LDS so that C is written in 16-byte
//    coalesced chunks.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;     // 8 waves: two per SIMD, so one wave's MFMAs cover the other's waits
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 256;            // B rows per tile (SwiGLU: 128 gate rows + 128 up rows)
constexpr int kBK = 64;             // K granularity the launch requires (K % 64 == 0)
// LDS pipeline geometry per tile height. The global->LDS path streams at ~53 B/clk per CU
// (measured on MI355X), so the largest tiles matter most: 256x256 tiles need ~31 B/clk at
// full MFMA rate against ~47 B/clk for 128x256. 256-row tiles use K slices of 32 (64-byte
// LDS rows) in a 4-deep ring of 32 KiB; smaller tiles use K slices of 64 (128-byte rows) in a
// 3-deep ring of up to 48 KiB. Stage = (BM rows of A + 256 rows of B) x row bytes.
template <int BM>
struct Pipe {
    static constexpr int BK = BM >= 256 ? 32 : 64;
    static constexpr int kRowBytes = BK * 2;
    static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per LDS row
    static constexpr int kStages = BM >= 256 ? 4 : 3;
    static constexpr int kStageBytes = (BM + kBN) * kRowBytes;
};
constexpr int kPipeBytes = 3 * (128 + kBN) * 128;           // 144 KiB (>= 4 x 32 KiB)
constexpr int kMaxGroups = 4095;
constexpr int kLdsBytes = kPipeBytes + (kMaxGroups + 1) * 4;   // 160 KiB
constexpr int kSuper = 4;           // column tiles per supertile

// 16-byte chunk c of LDS row r lives at slot c ^ swz(r). Chosen from measurements on gfx950
// of ds_read_b128 fragment reads (16 or 32 rows at one chunk): with 128-byte rows,
// (r >> 1) & 7 is conflict free (~230 B/clk/CU) for both 16x16 and 32x32 fragments (r & 7
// conflicts 2-way for 32 rows); with 64-byte rows, 32x32 fragments need (r >> 2) & 3 and
// 16x16 fragments (r >> 1) & 3 (each alternative conflicts 2-way).
template <int CHUNKS, int MS>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CHUNKS == 8) return (row >> 1) & 7;
    else if constexpr (MS == 32) return (row >> 2) & 3;
    else return (row >> 1) & 3;
}

// Tile height of a group with m rows. 256-row tiles need a bf16 C (their fp32 staging tile
// would not fit in LDS), so `max_bm` is 128 for fp32 output.
__device__ __forceinline__ int bm_of_rows(int m, int max_bm) {
    return m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : (m <= 192 || max_bm < 256) ? 128 : 256;
}

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
    int K;
    int NT;         // column tiles per group
    const char* A;
    int64_t lda;
    int64_t A_rows;
    const int32_t* a_rows;
    const char* B;
    int64_t ldb;
    int64_t b_stride;
    char* C;
    int64_t ldc;
    int c_f32;
    int max_bm;     // largest tile height used (128 when C is fp32)
    char* aux;
    int64_t ld_aux;
    const int32_t* tile_start;   // [G+1] in workspace
};

// ---------------------------------------------------------------------------------------
// schedule: tile_start[g] = sum over groups < g of ceil(m_g / BM_g) * NT
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets, int G, int M,
                                                             int NT, int max_bm, int32_t* __restrict__ tile_start) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += 1024) {
        const int g = g0 + tid;
        int tiles = 0;
        if (g < G) {
            int b, e;
            group_rows(offsets, g, M, b, e);
            const int m = e - b;
            tiles = m > 0 ? cdiv(m, bm_of_rows(m, max_bm)) * NT : 0;
        }
        int incl = tiles;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int wbase = carry_s;
        for (int w = 0; w < wave; ++w) wbase += wsum[w];
        if (g < G) tile_start[g] = wbase + incl - tiles;
        __syncthreads();
        if (tid == 1023) carry_s = wbase + incl;
        __syncthreads();
    }
    if (tid == 0) tile_start[G] = carry_s;
}

// ---------------------------------------------------------------------------------------
// one output tile of BM rows x (256 B-rows) for group g
// ---------------------------------------------------------------------------------------
// The two bf16 MFMA shapes used: operand fragment = one 16-byte LDS chunk per lane; the
// output tile is MS x MS with `out_row/out_col` giving the position of accumulator element r.
// Measured on MI355X from registers: 32x32x16 sustains ~2.28 PFLOP/s with 8 accumulators,
// 16x16x32 at most ~1.95, so the 64- and 128-row tiles use 32x32x16.
template <int MS>
struct Mfma;
template <>
struct Mfma<16> {
    using acc_t = f32x4;
    static constexpr int K = 32;         // contraction per instruction
    static constexpr int NACC = 4;       // accumulator floats per lane
    static __device__ __forceinline__ acc_t zero() { return acc_t{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 16; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 4 + lane / 16; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (lane / 16) * 4 + r; }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 16; }
};
template <>
struct Mfma<32> {
    using acc_t = f32x16;
    static constexpr int K = 16;
    static constexpr int NACC = 16;
    static __device__ __forceinline__ acc_t zero() {
        acc_t z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        return z;
    }
    static __device__ __forceinline__ acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int frag_row(int lane) { return lane % 32; }
    static __device__ __forceinline__ int frag_chunk(int lane, int ks) { return ks * 2 + lane / 32; }
    static __device__ __forceinline__ int out_row(int lane, int r) { return (r / 4) * 8 + (lane / 32) * 4 + (r % 4); }
    static __device__ __forceinline__ int out_col(int lane) { return lane % 32; }
};

template <int BM, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, char* lds, int g, int mt, int nt) {
    using PG = Pipe<BM>;
    constexpr int WM = (BM == 16) ? 1 : 2;    // wave grid: WM x WN = 8 waves
    constexpr int WN = kWaves / WM;
    constexpr int MS = (BM / WM >= 32) ? 32 : 16;   // MFMA tile edge
    using MF = Mfma<MS>;
    constexpr int RB = PG::kRowBytes;
    constexpr int CH = PG::kChunks;
    constexpr int ROWS_PER_INSTR = 1024 / RB;     // LDS rows filled by one 1 KiB DMA instruction
    constexpr int NKS = PG::BK / MF::K;          // MFMA k-steps per pipeline stage
    constexpr int WTM = BM / WM;              // rows per wave
    constexpr int WTN = kBN / WN;             // B rows (tile columns) per wave
    constexpr int MI = WTM / MS;
    constexpr int NI = WTN / MS;
    constexpr int A_INSTR = BM / ROWS_PER_INSTR;        // 1 KiB DMA instructions for the A slice
    constexpr int A_PER_WAVE = cdiv(A_INSTR, kWaves);
    constexpr int B_PER_WAVE = kBN / ROWS_PER_INSTR / kWaves;
    constexpr int BN_OUT = SWIGLU ? kBN / 2 : kBN;
    constexpr int kStages = PG::kStages;
    constexpr int kStageBytes = PG::kStageBytes;
    static_assert(kStages * kStageBytes <= kPipeBytes, "pipeline exceeds its LDS budget");
    static_assert(!SWIGLU || NI % 2 == 0, "SwiGLU needs gate and up fragments in every wave");

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    int row_begin, row_end;
    group_rows(p.offsets, g, p.M, row_begin, row_end);
    const int r0 = row_begin + mt * BM;                   // first C row of the tile
    const int n0 = nt * BN_OUT;                           // first output column

    // per-lane global source pointers for the DMA loads (fixed for the whole K loop);
    // lane l of an instruction fills LDS row (instr * ROWS_PER_INSTR + l / CH), slot l % CH
    const char* a_src[A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
        const int instr = wave + kWaves * i;
        const int row = instr * ROWS_PER_INSTR + lane / CH;
        const int chunk = (lane % CH) ^ swz<CH, MS>(row);
        int r = min(r0 + row, row_end - 1);
        int64_t ar = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
        ar = ar < 0 ? 0 : (ar >= p.A_rows ? p.A_rows - 1 : ar);
        a_src[i] = p.A + (ar * p.lda + chunk * 8) * 2;
    }
    const char* b_src[B_PER_WAVE];
    const char* bg = p.B + (int64_t)g * p.b_stride * 2;
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
        const int instr = wave * B_PER_WAVE + i;
        const int rho = instr * ROWS_PER_INSTR + lane / CH;   // LDS row of the B slice
        const int chunk = (lane % CH) ^ swz<CH, MS>(rho);
        int grow;
        if (SWIGLU) {
            const int wnb = rho / WTN, within = rho % WTN;
            const int half = within / (WTN / 2), idx = within % (WTN / 2);
            const int col = min(n0 + wnb * (WTN / 2) + idx, p.N - 1);
            grow = half * p.N + col;
        } else {
            grow = min(n0 + rho, p.N - 1);
        }
        b_src[i] = bg + ((int64_t)grow * p.ldb + chunk * 8) * 2;
    }

    auto issue = [&](int kt) {
        char* st = lds + (kt % kStages) * kStageBytes;
        const int64_t koff = (int64_t)kt * RB;
#pragma unroll
        for (int i = 0; i < A_PER_WAVE; ++i) {
            const int instr = wave + kWaves * i;
            if constexpr (A_INSTR % kWaves == 0) load_lds16(a_src[i] + koff, st + instr * 1024);
            else if (instr < A_INSTR) load_lds16(a_src[i] + koff, st + instr * 1024);
        }
        char* stb = st + BM * RB;
#pragma unroll
        for (int i = 0; i < B_PER_WAVE; ++i) load_lds16(b_src[i] + koff, stb + (wave * B_PER_WAVE + i) * 1024);
    };

    typename MF::acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = MF::zero();

    const int nk = p.K / PG::BK;
    // some waves issue no A load when BM < 64; the wait count uses the smallest
    // per-wave load count so that every wave is sure its own stage kt has landed
    constexpr int LOADS_MIN = B_PER_WAVE + A_INSTR / kWaves;
    static_assert((kStages - 2) * LOADS_MIN < 64, "vmcnt range");

    // per-lane LDS byte offsets of the MFMA fragments (fixed for the whole tile)
    int a_off[NKS][MI], b_off[NKS][NI];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int chunk = MF::frag_chunk(lane, ks);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int row = wm * WTM + i * MS + MF::frag_row(lane);
            a_off[ks][i] = row * RB + ((chunk ^ swz<CH, MS>(row)) << 4);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int row = wn * WTN + j * MS + MF::frag_row(lane);
            b_off[ks][j] = BM * RB + row * RB + ((chunk ^ swz<CH, MS>(row)) << 4);
        }
    }
    // Fragments are double-buffered in registers: the LDS reads of k-step ks+1 are issued
    // before the MFMAs of k-step ks, so LDS latency overlaps matrix work.
    auto compute = [&](int kt) {
        const char* st = lds + (kt % kStages) * kStageBytes;
        bf16x8 af[2][MI], bfr[2][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(st + a_off[0][i]);
#pragma unroll
        for (int j = 0; j < NI; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8*>(st + b_off[0][j]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            if (ks + 1 < NKS) {
#pragma unroll
                for (int i = 0; i < MI; ++i) af[nxt][i] = *reinterpret_cast<const bf16x8*>(st + a_off[ks + 1][i]);
#pragma unroll
                for (int j = 0; j < NI; ++j) bfr[nxt][j] = *reinterpret_cast<const bf16x8*>(st + b_off[ks + 1][j]);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of the MFMAs below
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = MF::run(af[cur][i], bfr[cur][j], acc[i][j]);
        }
    };

    // Ring of kStages LDS stages: stages kt+1 .. kt+kStages-2 stream in while stage kt is
    // multiplied. Before stage kt is read, this wave's loads of the later stages may still be
    // pending (LOADS_MIN each); the barrier then makes every wave's loads of stage kt visible
    // and guarantees the buffer refilled next (read in iteration kt-1) is no longer in use.
    lds_barrier();   // the previous tile's epilogue may still read LDS
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) issue(s);
    int kt = 0;
    for (; kt + kStages - 1 < nk; ++kt) {
        wait_vm_lgkm0<(kStages - 2) * LOADS_MIN>();
        lds_barrier();
        issue(kt + kStages - 1);
        compute(kt);
    }
    // tail: no more stages to issue; stages after kt still in flight = nk - 1 - kt
    for (; kt < nk; ++kt) {
        const int pending = nk - 1 - kt;
        if constexpr (kStages >= 4) {
            if (pending >= 2) wait_vm_lgkm0<2 * LOADS_MIN>();
            else if (pending == 1) wait_vm_lgkm0<LOADS_MIN>();
            else wait_vm_lgkm0<0>();
        } else {
            if (pending >= 1) wait_vm_lgkm0<LOADS_MIN>();
            else wait_vm_lgkm0<0>();
        }
        lds_barrier();
        compute(kt);
    }

    // ---- epilogue: values -> LDS (output dtype) -> 16-byte coalesced global stores ----
    wait_vm_lgkm0<0>();
    lds_barrier();
    const int esize = p.c_f32 ? 4 : 2;
    const int pitch = BN_OUT * esize + 16;
    const int rows_valid = min(BM, row_end - r0);
    constexpr int NO = SWIGLU ? NI / 2 : NI;       // output fragments per wave row block
    constexpr int WOUT = SWIGLU ? WTN / 2 : WTN;   // output columns per wave
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
    for (int c = tid; c < BM * chunks_per_row; c += kThreads) {
        const int row = c / chunks_per_row, ch = c % chunks_per_row;
        const int col = n0 + ch * cols_per_chunk;
        if (row < rows_valid && col < p.N) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * pitch + ch * 16);
            *reinterpret_cast<u32x4*>(p.C + ((int64_t)(r0 + row) * p.ldc + col) * esize) = v;
        }
    }
}

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int32_t* ts = reinterpret_cast<int32_t*>(lds + kPipeBytes);
    for (int g = threadIdx.x; g <= p.G; g += kThreads) ts[g] = p.tile_start[g];
    __syncthreads();
    const int total = ts[p.G];
    // XCD-aware slot: the hardware deals workgroups round-robin over the 8 XCDs, so give the
    // workgroups of one XCD consecutive slots (and hence consecutive tiles in each round)
    const int nxcd = (gridDim.x % 8 == 0) ? 8 : 1;
    const int per_xcd = gridDim.x / nxcd;
    const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
    for (int tile = slot; tile < total; tile += gridDim.x) {
        // group = last g with ts[g] <= tile
        int lo = 0, hi = p.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ts[mid] <= tile) lo = mid;
            else hi = mid - 1;
        }
        const int g = lo;
        const int L = tile - ts[g];
        int gb, ge;
        group_rows(p.offsets, g, p.M, gb, ge);
        const int m = ge - gb;
        const int bm = bm_of_rows(m, p.max_bm);
        const int MT = cdiv(m, bm);
        const int NT = p.NT;
        const int full = NT / kSuper;
        int mt, nt;
        if (L < full * MT * kSuper) {
            const int s = L / (MT * kSuper), rem = L % (MT * kSuper);
            mt = rem / kSuper;
            nt = s * kSuper + rem % kSuper;
        } else {
            const int rem = L - full * MT * kSuper, w = NT - full * kSuper;
            mt = rem / w;
            nt = full * kSuper + rem % w;
        }
        switch (bm) {
            case 16: gemm_tile<16, SWIGLU>(p, lds, g, mt, nt); break;
            case 32: gemm_tile<32, SWIGLU>(p, lds, g, mt, nt); break;
            case 64: gemm_tile<64, SWIGLU>(p, lds, g, mt, nt); break;
            default: gemm_tile<128, SWIGLU>(p, lds, g, mt, nt); break;
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

bool set_lds_attr() {
    static bool done[2] = {false, false};
    if (!done[0]) {
        if (hipFuncSetAttribute((const void*)gemm_bf16_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsBytes) != hipSuccess)
            return false;
        done[0] = true;
    }
    if (!done[1]) {
        if (hipFuncSetAttribute((const void*)gemm_bf16_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsBytes) != hipSuccess)
            return false;
        done[1] = true;
    }
    return true;
}

}  // namespace
}  // namespace moe

size_t moe_gemm_workspace_bytes(int32_t G) {
    if (G < 1) G = 1;
    return (((size_t)G + 1) * 4 + 255) & ~size_t(255);
}

extern "C" moe_status_t moe_grouped_gemm(const moe_gemm_args_t* a, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    if (!a) return MOE_EINVAL;
    if (a->G < 1 || a->G > moe::kMaxGroups || !a->offsets) return MOE_EINVAL;
    if (a->M < 0 || a->N <= 0 || a->K <= 0 || a->N % 8 != 0 || a->N > (1 << 24) || a->K > (1 << 24))
        return MOE_EINVAL;
    if (a->M > INT32_MAX / 2) return MOE_EINVAL;
    if (a->epilogue != MOE_EPI_NONE && a->epilogue != MOE_EPI_SWIGLU) return MOE_EINVAL;
    if (a->a_dtype != a->b_dtype) return MOE_ENOTSUP;
    if (a->a_dtype != MOE_BF16 && a->a_dtype != MOE_F32) return MOE_ENOTSUP;
    if (a->c_dtype != MOE_BF16 && a->c_dtype != MOE_F32) return MOE_ENOTSUP;
    if (a->a_dtype == MOE_F32 && a->c_dtype != MOE_F32) return MOE_ENOTSUP;
    if (a->M == 0) return MOE_OK;
    if (!a->A || !a->B || !a->C || a->A_rows <= 0) return MOE_EINVAL;
    // groups' B matrices are only read, so they may overlap (e.g. K slices of one matrix)
    if (a->lda < a->K || a->ldb < a->K || a->ldc < a->N || a->b_group_stride < 0) return MOE_EINVAL;
    if (a->aux && (a->epilogue != MOE_EPI_SWIGLU || a->ld_aux < 2 * a->N)) return MOE_EINVAL;
    if (!workspace || workspace_bytes < moe_gemm_workspace_bytes(a->G)) return MOE_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;

    moe::GemmParams p;
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
    // 256-row tiles (4-stage, 32-wide K slices) measured faster on a square 8192^3 product but
    // slower on the DeepSeek-V3 and Mixtral expert shapes, so the launch stops at 128 rows.
    p.max_bm = 128;
    p.aux = (char*)a->aux;
    p.ld_aux = a->ld_aux;
    p.tile_start = (const int32_t*)workspace;
    const bool swiglu = a->epilogue == MOE_EPI_SWIGLU;

    if (a->a_dtype == MOE_F32) {
        p.NT = 0;
        const int64_t n = a->M * a->N;
        hipLaunchKernelGGL(moe::gemm_f32_kernel, dim3((unsigned)moe::cdiv<int64_t>(n, 256)), dim3(256), 0, s, p,
                           a->M, swiglu ? 1 : 0);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // bf16 MFMA path
    if (a->K % moe::kBK != 0) return MOE_EINVAL;
    if (!moe_aligned16(a->A) || !moe_aligned16(a->B) || !moe_aligned16(a->C)) return MOE_EINVAL;
    if (a->lda % 8 || a->ldb % 8 || a->ldc % 8 || a->b_group_stride % 8) return MOE_EINVAL;
    if (a->aux && (!moe_aligned16(a->aux) || a->ld_aux % 8)) return MOE_EINVAL;
    const int bn_out = swiglu ? moe::kBN / 2 : moe::kBN;
    p.NT = (int)moe::cdiv<int64_t>(a->N, bn_out);
    if (!moe::set_lds_attr()) return MOE_EHIP;
    hipLaunchKernelGGL(moe::gemm_schedule_kernel, dim3(1), dim3(1024), 0, s, a->offsets, a->G, p.M, p.NT, p.max_bm,
                       (int32_t*)workspace);
    MOE_CHECK_LAUNCH();
    // enough persistent workgroups to fill every CU, never more than the tile bound
    const int64_t bound = (a->M / 16 + a->G) * (int64_t)p.NT;
    const int64_t grid = std::min<int64_t>((int64_t)moe::num_cus(), std::max<int64_t>(bound, 1));
    if (swiglu)
        hipLaunchKernelGGL(moe::gemm_bf16_kernel<true>, dim3((unsigned)grid), dim3(moe::kThreads), moe::kLdsBytes, s, p);
    else
        hipLaunchKernelGGL(moe::gemm_bf16_kernel<false>, dim3((unsigned)grid), dim3(moe::kThreads), moe::kLdsBytes, s, p);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

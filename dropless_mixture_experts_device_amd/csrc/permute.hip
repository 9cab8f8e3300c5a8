// moe_permute: per-expert histogram, group offsets, stable permutation and row gather, all
// on the device with a fixed launch shape, so group sizes never reach the host.
//
// [Blog] "Optimisation 2": dispatch reorders tokens locally so that each expert's tokens are
// contiguous; combine restores the order. [Blog] "Optimisation 1": the counts are never
// copied to the host (that copy sat on the critical path of the per-expert GEMM loop).
//
// Deterministic counting sort without order-dependent atomics:
//   1. mask:  for every 64-token sub-tile and expert, a 64-bit mask of the tokens that chose
//             the expert (built with LDS atomic OR, whose result does not depend on order),
//             plus exclusive prefix counts of the 16 sub-tiles of each 1024-token tile.
//   2. scan:  per expert, exclusive prefix over tiles; across experts, the group offsets.
//   3. place: row(t, j) = base[tile][e] + subprefix[tile][sub][e]
//                         + popcount(mask[tile][sub][e] & bits below t)
//             then copy x[t] to its k rows (x is read once per token).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSub = 64;                 // tokens per mask word
constexpr int kSubPerTile = 16;
constexpr int kTile = kSub * kSubPerTile; // 1024 tokens per histogram tile
constexpr int kPermThreads = 256;
// 16-byte chunks of x[t] a lane holds before the stores: 14 covers a 7,168-column bf16 row
// in one pass, so each of its copies goes out as one 14 KiB burst (the DeepSeek-V3 gather
// 0.231 -> 0.224 ms against 4 chunks, 0.228 with 8)
#ifndef MOE_PERMUTE_UNROLL
#define MOE_PERMUTE_UNROLL 14
#endif

struct PermWs {
    uint64_t* mask;      // [nsub][E]
    int32_t* subprefix;  // [nsub][E]   exclusive prefix inside the tile
    int32_t* base;       // [ntile][E]  tile counts, then absolute bases
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__host__ __device__ inline PermWs perm_ws(void* ws, int64_t T, int E) {
    const int64_t nsub = cdiv<int64_t>(T, kSub), ntile = cdiv<int64_t>(T, kTile);
    char* p = (char*)ws;
    PermWs w;
    w.mask = (uint64_t*)p;
    p += align256(nsub * E * sizeof(uint64_t));
    w.subprefix = (int32_t*)p;
    p += align256(nsub * E * sizeof(int32_t));
    w.base = (int32_t*)p;
    (void)ntile;
    return w;
}

// One workgroup of kMaskThreads per 1024-token tile. Each thread first loads all of its
// (token, slot) pairs' expert ids (independent loads in flight together), then ORs the
// token bits into the LDS masks.
constexpr int kMaskThreads = 1024;
constexpr int kMaskPer = 16;   // pairs per thread per pass (k <= 16: one pass per tile)

__global__ __launch_bounds__(kMaskThreads) void perm_mask_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                                 int E, int k, PermWs ws) {
    extern __shared__ unsigned long long smask[];   // [kSubPerTile][E]
    const int tile = blockIdx.x;
    for (int i = threadIdx.x; i < kSubPerTile * E; i += kMaskThreads) smask[i] = 0ull;
    __syncthreads();
    const int t_begin = tile * kTile;
    const int npairs = min(kTile, T - t_begin) * k;
    const int32_t* src = topk_idx + (int64_t)t_begin * k;
    for (int p0 = 0; p0 < npairs; p0 += kMaskThreads * kMaskPer) {
        int ev[kMaskPer];
#pragma unroll
        for (int u = 0; u < kMaskPer; ++u) {
            const int p = p0 + u * kMaskThreads + threadIdx.x;
            ev[u] = p < npairs ? src[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kMaskPer; ++u) {
            const int p = p0 + u * kMaskThreads + threadIdx.x;
            const int tl = p / k;
            if ((unsigned)ev[u] < (unsigned)E) atomicOr(&smask[(tl / kSub) * E + ev[u]], 1ull << (tl % kSub));
        }
    }
    __syncthreads();
    const int nsub_here = cdiv(min(kTile, T - t_begin), kSub);
    const int64_t sub0 = (int64_t)tile * kSubPerTile;
    for (int e = threadIdx.x; e < E; e += kMaskThreads) {
        int run = 0;
        for (int s = 0; s < nsub_here; ++s) {
            const unsigned long long m = smask[s * E + e];
            ws.mask[(sub0 + s) * E + e] = m;
            ws.subprefix[(sub0 + s) * E + e] = run;
            run += __popcll(m);
        }
        ws.base[(int64_t)tile * E + e] = run;
    }
}

// One workgroup: per-expert prefix over tiles, then the exclusive scan over experts.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int T, int E, int k, int shared_group, PermWs ws,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int wsum[16];
    const int ntile = cdiv(T, kTile);
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // 8 tiles' counts are loaded together before any is overwritten, so their latencies overlap
        constexpr int U = 8;
        for (int t0 = 0; t0 < ntile; t0 += U) {
            int c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) c[u] = t0 + u < ntile ? ws.base[(int64_t)(t0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (t0 + u < ntile) ws.base[(int64_t)(t0 + u) * E + e] = run;
                run += c[u];
            }
        }
    }
    // exclusive scan of run over e (E <= 1024) with wave prefix sums
    const int lane = e % kWave, wave = e / kWave;
    int incl = run;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const int o = __shfl_up(incl, s, kWave);
        if (lane >= s) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    const int excl = wbase + incl - run;
    if (e < E) offsets[e] = excl;
    if (e == 0) {
        offsets[E] = T * k;
        if (shared_group) offsets[E + 1] = T * k + T;
    }
    if (e < E) {
        for (int t = 0; t < ntile; ++t) ws.base[(int64_t)t * E + e] += excl;
    }
}

// One wave per token: its k rows, the index maps, and the copy of x[t] to every row.
template <int ESIZE>
__global__ __launch_bounds__(kPermThreads) void perm_place_kernel(
    const int32_t* __restrict__ topk_idx, const char* __restrict__ x, int T, int d, int E, int k,
    int shared_group, PermWs ws, int32_t* __restrict__ row_of, int32_t* __restrict__ src_token,
    char* __restrict__ x_perm) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * (kPermThreads / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const int TK = T * k;
    int row = -1;
    if (lane < k) {
        int e = topk_idx[(int64_t)t * k + lane];
        e = min(max(e, 0), E - 1);
        const int tile = t / kTile, sub = t / kSub, bit = t % kSub;
        const unsigned long long m = ws.mask[(int64_t)sub * E + e];
        const unsigned long long below = bit ? (m & ((1ull << bit) - 1ull)) : 0ull;
        row = ws.base[(int64_t)tile * E + e] + ws.subprefix[(int64_t)sub * E + e] + __popcll(below);
        row = min(max(row, 0), TK - 1);
        row_of[(int64_t)t * k + lane] = row;
        src_token[row] = t;
    }
    if (shared_group && lane == 0) src_token[TK + t] = t;
    if (x_perm == nullptr) return;
    const int nrows = k + (shared_group ? 1 : 0);
    const int nchunk = d * ESIZE / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)t * d * ESIZE);
    constexpr int U = MOE_PERMUTE_UNROLL;   // 16-byte chunks per lane in flight before the stores
    for (int c0 = lane; c0 < nchunk; c0 += kWave * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave;
            if (c < nchunk) v[u] = src[c];
        }
        for (int j = 0; j < nrows; ++j) {
            const int rj = (j < k) ? __shfl(row, j, kWave) : TK + t;
            u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (int64_t)rj * d * ESIZE);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave;
                if (c < nchunk) __builtin_nontemporal_store(v[u], dst + c);   // x_perm is not read here again
            }
        }
    }
}

}  // namespace
}  // namespace moe

size_t moe_permute_workspace_bytes(int64_t T, int32_t E) {
    if (T <= 0 || E <= 0) return 256;
    const int64_t nsub = moe::cdiv<int64_t>(T, moe::kSub), ntile = moe::cdiv<int64_t>(T, moe::kTile);
    return moe::align256(nsub * E * 8) + moe::align256(nsub * E * 4) + moe::align256(ntile * E * 4);
}

extern "C" moe_status_t moe_permute(const void* x, int32_t dtype, const int32_t* topk_idx, int64_t T, int64_t d,
                                    int32_t E, int32_t k, int32_t shared_group, int32_t* offsets,
                                    int32_t* row_of, int32_t* src_token, void* x_perm, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (T < 0 || E < 1 || E > 512 || k < 1 || k > 16 || k > E) return MOE_EINVAL;
    if ((T + 1) * (int64_t)(k + 1) > INT32_MAX) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (T > 0 && (!topk_idx || !row_of || !src_token)) return MOE_EINVAL;
    int esize = 0;
    if (x_perm != nullptr) {
        if (dtype == MOE_BF16) esize = 2;
        else if (dtype == MOE_F32) esize = 4;
        else return MOE_ENOTSUP;
        if (d <= 0 || d % 8 != 0 || d > INT32_MAX / 16) return MOE_EINVAL;
        if (T > 0 && (!x || !moe_aligned16(x) || !moe_aligned16(x_perm))) return MOE_EINVAL;
    }
    if (!workspace || workspace_bytes < moe_permute_workspace_bytes(T, E)) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
#if MOE_DEBUG
    {
        // expert ids within [0, E) and distinct within each token
        std::vector<int32_t> ids;
        if (!moe_debug_fetch_i32(topk_idx, T * k, s, ids)) return MOE_EHIP;
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j) {
                const int32_t e = ids[t * k + j];
                if (e < 0 || e >= E) return MOE_EINVAL;
                for (int i = 0; i < j; ++i)
                    if (ids[t * k + i] == e) return MOE_EINVAL;
            }
    }
#endif
    const int Ti = (int)T;
    moe::PermWs ws = moe::perm_ws(workspace, T, E);
    if (T > 0) {
        const int ntile = moe::cdiv(Ti, moe::kTile);
        hipLaunchKernelGGL(moe::perm_mask_kernel, dim3(ntile), dim3(moe::kMaskThreads),
                           moe::kSubPerTile * E * sizeof(unsigned long long), s, topk_idx, Ti, E, k, ws);
        MOE_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(moe::perm_scan_kernel, dim3(1), dim3(1024), 0, s, Ti, E, k, shared_group ? 1 : 0, ws,
                       offsets);
    MOE_CHECK_LAUNCH();
    if (T > 0) {
        const dim3 grid(moe::cdiv(Ti, moe::kPermThreads / moe::kWave));
        if (esize == 4)
            hipLaunchKernelGGL(moe::perm_place_kernel<4>, grid, dim3(moe::kPermThreads), 0, s, topk_idx,
                               (const char*)x, Ti, (int)d, E, k, shared_group ? 1 : 0, ws, row_of, src_token,
                               (char*)x_perm);
        else
            hipLaunchKernelGGL(moe::perm_place_kernel<2>, grid, dim3(moe::kPermThreads), 0, s, topk_idx,
                               (const char*)x, Ti, (int)(x_perm ? d : 0), E, k, shared_group ? 1 : 0, ws, row_of,
                               src_token, (char*)x_perm);
        MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
}

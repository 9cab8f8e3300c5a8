// moe_route: router projection (bf16 MFMA, fp32 accumulate), expert bias, top-k selection
// and normalised routing weights. Small layers: one fused kernel per 32-token tile. Large
// layers (the skinny projection would fill too few CUs): the projection as K-split partial
// sums on the grouped-GEMM kernel, then one pass that sums them in a fixed order, adds the
// bias and selects (two launches).
//
// [Blog] opening section: a learnable router picks each token's top-K experts;
// [Blog] "Optimisation 2": a single fused router kernel assigns the experts.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteBT = 32;       // tokens per workgroup
constexpr int kRouteThreads = 256; // 4 waves

// Map a float to an unsigned key whose unsigned order is the float order (-0 folded to +0).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide max of a 32-bit value, returned to every lane. DPP lane moves stay in the VALU
// (no LDS round trip): pairs, quads, then rotations inside each 16-lane row give every lane
// its row's max; two row broadcasts fold the rows so lane 63 holds the wave max. Lanes
// outside a step's row mask keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
    return o > v ? o : v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_step<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_max_step<0x124, 0xF>(v);   // row_ror:4
    v = dpp_max_step<0x128, 0xF>(v);   // row_ror:8
    v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float key_of_ordered(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Top-k over keys held in LDS ([BT][pitch] floats, bias already added). Each wave handles
// tokens wave, wave+4, ... of the tile; lane l holds experts l, 64+l, ... as order-preserving
// 32-bit codes (0 = absent or already taken; every finite key codes above 0). One round per
// selection: the wave max of the codes, then the lowest expert id holding it (ballots in
// expert order), which is removed. Selection order: larger key first, equal keys -> lower
// expert id. Lane j keeps the j-th selection and writes it with its weight.
template <int NQ, int BT = kRouteBT>
__device__ void topk_tile(const float* keys, int pitch, int t0, int T, int E, int k, int score,
                          int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    for (int tl = wave; tl < BT; tl += kRouteThreads / kWave) {
        const int t = t0 + tl;
        if (t >= T) break;
        uint32_t cand[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = q * kWave + lane;
            cand[q] = (e < E) ? ordered_bits(keys[tl * pitch + e]) : 0u;
        }
        uint32_t my_code = 0u, code0 = 0u;
        int my_e = 0;
        for (int j = 0; j < k; ++j) {
            uint32_t m = cand[0];
#pragma unroll
            for (int q = 1; q < NQ; ++q) m = cand[q] > m ? cand[q] : m;
            m = wave_max_u32(m);
            int win = -1;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const unsigned long long b = __ballot(cand[q] == m);
                if (win < 0 && b != 0ull) win = q * kWave + __builtin_ctzll(b);
            }
            win = min(max(win, 0), E - 1);   // in range even for non-finite keys (unsupported)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (q * kWave + lane == win) cand[q] = 0u;
            if (lane == j) {
                my_code = m;
                my_e = win;
            }
            if (j == 0) code0 = m;
        }
        // weights: lane j < k forms its term; the normaliser adds the terms in the order j = 0 .. k-1
        const float key0 = key_of_ordered(code0), kj = key_of_ordered(my_code);
        float z = 0.f;
        if (lane < k) z = (score == MOE_SOFTMAX) ? expf(kj - key0) : 1.0f / (1.0f + expf(-kj));
        float sum = 0.f;
        for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
        if (lane < k) {
            topk_idx[(int64_t)t * k + lane] = my_e;
            topk_w[(int64_t)t * k + lane] = z / sum;
        }
    }
}

// bf16 router: each wave owns NTW*16 experts and all 32 tokens of the tile; A (tokens) and
// B (router rows) fragments are loaded straight from global memory into registers (no LDS:
// no operand is shared between waves except the small token tile, which stays in L1/L2).
template <int NTW, int NQ>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias,
    int T, int d, int E, int k, int score, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ keys_out) {
    constexpr int EPAD = NTW * 16 * 4;
    constexpr int PITCH = EPAD + 4;
    __shared__ float keys[kRouteBT * PITCH];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kRouteBT;
    const int ebase = wave * NTW * 16;
    const int sub = lane / 16;   // which 8-element k chunk of the 32-wide step
    const int r16 = lane % 16;

    const uint16_t* arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int t = t0 + i * 16 + r16;
        t = t < T ? t : T - 1;
        arow[i] = x + (int64_t)t * d;
    }
    const uint16_t* brow[NTW];
    bool bval[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        int e = ebase + j * 16 + r16;
        bval[j] = e < E;
        brow[j] = w + (int64_t)(e < E ? e : E - 1) * d;
    }
    f32x4 acc[2][NTW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int U = 4;   // k-steps of 32 issued together
    const bf16x8 zero8 = {};
    for (int k0 = 0; k0 < d; k0 += 32 * U) {
        bf16x8 af[U][2], bfr[U][NTW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * 32 + sub * 8;
            const bool in = kk < d;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[u][i] = in ? *reinterpret_cast<const bf16x8*>(arow[i] + kk) : zero8;
#pragma unroll
            for (int j = 0; j < NTW; ++j)
                bfr[u][j] = (in && bval[j]) ? *reinterpret_cast<const bf16x8*>(brow[j] + kk) : zero8;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][i], bfr[u][j], acc[i][j], 0, 0, 0);
    }
    // logits + bias -> LDS; the 16x16 output tile puts rows 4*(lane/16)+r, column lane%16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int e = ebase + j * 16 + r16;
            const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) keys[(i * 16 + sub * 4 + r) * PITCH + e] = acc[i][j][r] + b;
        }
    __syncthreads();
    if (keys_out != nullptr) {
        for (int idx = threadIdx.x; idx < kRouteBT * E; idx += kRouteThreads) {
            const int tl = idx / E, e = idx % E;
            if (t0 + tl < T) keys_out[(int64_t)(t0 + tl) * E + e] = keys[tl * PITCH + e];
        }
    }
    topk_tile<NQ>(keys, PITCH, t0, T, E, k, score, topk_idx, topk_w);
}

// fp32 router (small, correctness-oriented): plain fp32 FMA dot products, sequential in d.
template <int NQ>
__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias, int T,
    int d, int E, int k, int score, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ keys_out) {
    constexpr int PITCH = NQ * kWave + 4;
    __shared__ float keys[kRouteBT * PITCH];
    const int t0 = blockIdx.x * kRouteBT;
    for (int idx = threadIdx.x; idx < kRouteBT * E; idx += kRouteThreads) {
        const int tl = idx / E, e = idx % E;
        const int t = min(t0 + tl, T - 1);
        const float* xr = x + (int64_t)t * d;
        const float* wr = w + (int64_t)e * d;
        float s = 0.f;
        for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
        keys[tl * PITCH + e] = s + (bias != nullptr ? bias[e] : 0.f);
    }
    __syncthreads();
    if (keys_out != nullptr) {
        for (int idx = threadIdx.x; idx < kRouteBT * E; idx += kRouteThreads) {
            const int tl = idx / E, e = idx % E;
            if (t0 + tl < T) keys_out[(int64_t)(t0 + tl) * E + e] = keys[tl * PITCH + e];
        }
    }
    topk_tile<NQ>(keys, PITCH, t0, T, E, k, score, topk_idx, topk_w);
}

// ---- split-K router for large layers -------------------------------------------------------
// The projection x[T,d] . w_router[E,d]^T is a skinny GEMM (E <= 256 columns): with one
// 128-token tile per workgroup it fills only T/128 CUs. It therefore runs on the grouped-GEMM
// kernel as KS uniform groups, group s multiplying the s-th K slice of x and of w_router in
// place (every group has the same T rows, so no index, offsets or schedule are built). The
// fp32 partial logits are then summed in the fixed order s = 0..KS-1, the bias added, and the
// top-k taken.
constexpr int kRouteKS = 4;

__host__ __device__ inline size_t ralign(size_t v) { return (v + 255) & ~size_t(255); }

inline bool route_uses_split(int64_t T, int64_t d, int E) {
    return T >= 256 && E % 8 == 0 && d % (64 * kRouteKS) == 0;
}

// The split-K pass's selection: 16 lanes per token, 4 tokens per wave, 16 tokens per
// workgroup. Lane r of a token's group owns the experts 64q + 4r + i (i < 4, q < NQ): each of
// its loads is one 16-byte chunk of a partial-logit row, so the 16 lanes read 256 contiguous
// bytes. The KS partials of a chunk are loaded before any is summed, then summed in the
// order s = 0..KS-1 and the bias added, exactly as the keys are defined. Each selection round
// takes the 16-lane maximum of the order-preserving codes, then the 16-lane minimum of the
// expert ids holding it (equal keys -> lower expert id), and the owner removes it; lane j of
// the group keeps selection j. Row-wide (16-lane) reductions use DPP moves inside the row.
constexpr int kTopkTok = 16;   // tokens per workgroup of the split-K selection pass

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_min_step(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
    return o < v ? o : v;
}

// every lane gets the maximum (minimum) of its 16-lane row: quad swaps, then rotations by 4, 8
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = dpp_max_step<0xB1, 0xF>(v);
    v = dpp_max_step<0x4E, 0xF>(v);
    v = dpp_max_step<0x124, 0xF>(v);
    return dpp_max_step<0x128, 0xF>(v);
}

__device__ __forceinline__ uint32_t row_min_u32(uint32_t v) {
    v = dpp_min_step<0xB1>(v);
    v = dpp_min_step<0x4E>(v);
    v = dpp_min_step<0x124>(v);
    return dpp_min_step<0x128>(v);
}

template <int NQ>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float* __restrict__ partial,
                                                                   const float* __restrict__ bias, int T, int E,
                                                                   int k, int score, int32_t* __restrict__ topk_idx,
                                                                   float* __restrict__ topk_w,
                                                                   float* __restrict__ keys_out) {
    constexpr int P = 4 * NQ;   // candidates per lane
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int r = lane % 16, grp = lane / 16;
    const int t = blockIdx.x * kTopkTok + wave * 4 + grp;
    const int tc = min(t, T - 1);   // rows past T load the last token's row and write nothing
    f32x4 v[NQ][kRouteKS];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e0 = 64 * q + 4 * r;
        if (e0 < E) {
#pragma unroll
            for (int s = 0; s < kRouteKS; ++s)
                v[q][s] = *reinterpret_cast<const f32x4*>(partial + ((int64_t)s * T + tc) * E + e0);
        }
    }
    uint32_t code[P];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e0 = 64 * q + 4 * r;
        f32x4 key = {0.f, 0.f, 0.f, 0.f};
        if (e0 < E) {   // E % 4 == 0 on this path, so a chunk is wholly in or out
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sum = 0.f;
#pragma unroll
                for (int s = 0; s < kRouteKS; ++s) sum += v[q][s][i];
                key[i] = sum + (bias != nullptr ? bias[e0 + i] : 0.f);
            }
            if (keys_out != nullptr && t < T) *reinterpret_cast<f32x4*>(keys_out + (int64_t)t * E + e0) = key;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) code[4 * q + i] = e0 < E ? ordered_bits(key[i]) : 0u;
    }
    uint32_t my_code = 0u, code0 = 0u;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t m = code[0];
#pragma unroll
        for (int c = 1; c < P; ++c) m = code[c] > m ? code[c] : m;
        m = row_max_u32(m);
        uint32_t el = 0xFFFFFFFFu;   // this lane's lowest expert id holding the maximum
#pragma unroll
        for (int c = P - 1; c >= 0; --c)
            if (m != 0u && code[c] == m) el = (uint32_t)(64 * (c / 4) + 4 * r + c % 4);
        const uint32_t ew = row_min_u32(el);
        const int win = min(max((int)ew, 0), E - 1);   // in range even for non-finite keys (unsupported)
#pragma unroll
        for (int c = 0; c < P; ++c)
            if (64 * (c / 4) + 4 * r + c % 4 == win) code[c] = 0u;
        if (r == j) {
            my_code = m;
            my_e = win;
        }
        if (j == 0) code0 = m;
    }
    // weights: lane j < k of the group forms its term; the normaliser adds the terms in the order j = 0 .. k-1
    const float key0 = key_of_ordered(code0), kj = key_of_ordered(my_code);
    float z = 0.f;
    if (r < k) z = (score == MOE_SOFTMAX) ? expf(kj - key0) : 1.0f / (1.0f + expf(-kj));
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += __shfl(z, grp * 16 + j, kWave);
    if (t < T && r < k) {
        topk_idx[(int64_t)t * k + r] = my_e;
        topk_w[(int64_t)t * k + r] = z / sum;
    }
}

template <int NTW>
void launch_route_bf16(dim3 g, hipStream_t s, const void* x, const void* w, const float* b, int T, int d,
                       int E, int k, int score, int32_t* ti, float* tw, float* ko) {
    constexpr int NQ = (NTW * 64 + 63) / 64;
    hipLaunchKernelGGL((route_bf16_kernel<NTW, NQ>), g, dim3(kRouteThreads), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w, b, T, d, E, k, score, ti, tw, ko);
}

}  // namespace
}  // namespace moe

size_t moe_route_workspace_bytes(int64_t T, int64_t d, int32_t E) {
    if (T <= 0 || E <= 0 || !moe::route_uses_split(T, d, E)) return 0;
    return moe::ralign((size_t)moe::kRouteKS * T * E * 4);   // partial logits [KS*T, E] fp32
}

extern "C" moe_status_t moe_route(const void* x, const void* w_router, int32_t dtype, const float* bias,
                                  int64_t T, int64_t d, int32_t E, int32_t k, int32_t score,
                                  int32_t* topk_idx, float* topk_w, float* keys_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (T < 0 || d <= 0 || E < 1 || E > 256 || k < 1 || k > 16 || k > E) return MOE_EINVAL;
    if (d % 8 != 0 || T > INT32_MAX / 16 || d > INT32_MAX / 16) return MOE_EINVAL;
    if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_EINVAL;
    if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w) return MOE_EINVAL;
    if (!moe_aligned16(x) || !moe_aligned16(w_router)) return MOE_EINVAL;
    const bool split = dtype == MOE_BF16 && moe::route_uses_split(T, d, E);
    if (split && (!workspace || workspace_bytes < moe_route_workspace_bytes(T, d, E))) return MOE_EWORKSPACE;
    if (split && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)moe::cdiv<int64_t>(T, moe::kRouteBT));
    const int Ti = (int)T, di = (int)d;
    if (split) {
        float* partial = (float*)workspace;
        const moe_status_t st = moe_gemm_ksplit_f32(x, w_router, T, d, E, moe::kRouteKS, partial, s);
        if (st != MOE_OK) return st;
        const int nq = moe::cdiv(E, 64);
        const dim3 tgrid((unsigned)moe::cdiv<int64_t>(T, moe::kTopkTok));
        if (nq <= 1)
            hipLaunchKernelGGL((moe::route_topk_kernel<1>), tgrid, dim3(moe::kRouteThreads), 0, s, partial, bias, Ti, E,
                               k, score, topk_idx, topk_w, keys_out);
        else if (nq <= 2)
            hipLaunchKernelGGL((moe::route_topk_kernel<2>), tgrid, dim3(moe::kRouteThreads), 0, s, partial, bias, Ti, E,
                               k, score, topk_idx, topk_w, keys_out);
        else
            hipLaunchKernelGGL((moe::route_topk_kernel<4>), tgrid, dim3(moe::kRouteThreads), 0, s, partial, bias, Ti, E,
                               k, score, topk_idx, topk_w, keys_out);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    if (dtype == MOE_BF16) {
        const int ntw = moe::cdiv(E, 64);   // 16-expert tiles per wave, 4 waves
        switch (ntw) {
            case 1: moe::launch_route_bf16<1>(grid, s, x, w_router, bias, Ti, di, E, k, score, topk_idx, topk_w, keys_out); break;
            case 2: moe::launch_route_bf16<2>(grid, s, x, w_router, bias, Ti, di, E, k, score, topk_idx, topk_w, keys_out); break;
            default: moe::launch_route_bf16<4>(grid, s, x, w_router, bias, Ti, di, E, k, score, topk_idx, topk_w, keys_out); break;
        }
    } else {
        const int nq = moe::cdiv(E, 64);
        if (nq <= 1)
            hipLaunchKernelGGL((moe::route_f32_kernel<1>), grid, dim3(moe::kRouteThreads), 0, s, (const float*)x,
                               (const float*)w_router, bias, Ti, di, E, k, score, topk_idx, topk_w, keys_out);
        else
            hipLaunchKernelGGL((moe::route_f32_kernel<4>), grid, dim3(moe::kRouteThreads), 0, s, (const float*)x,
                               (const float*)w_router, bias, Ti, di, E, k, score, topk_idx, topk_w, keys_out);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

// Internal helpers shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

namespace moe {

constexpr int kWave = 64;

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (expcnt untouched). The gfx9 encoding keeps
// vmcnt in bits [3:0] and [15:14], expcnt in [6:4], lgkmcnt in [11:8].
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier that does NOT drain outstanding global->LDS loads (the fence inside
// __syncthreads would wait for every one of them). Callers wait for exactly the loads they
// need with wait_vm_lgkm0<N>() first. The empty asm statements stop the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes from global memory straight into LDS. Lane i of the wave writes LDS bytes
// [lds_wave_base + 16 i, +16); lds_wave_base must be the same for the whole wave.
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gptr, MOE_LDS(lds_wave_base), 16, 0, 0);
}

// 4 bytes from global memory into LDS: lane i writes LDS bytes [lds_wave_base + 4 i, +4).
__device__ __forceinline__ void load_lds4(const void* gptr, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gptr, MOE_LDS(lds_wave_base), 4, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <typename T>
__host__ __device__ constexpr T cdiv(T a, T b) { return (a + b - 1) / b; }

}  // namespace moe

#define MOE_CHECK_LAUNCH()                                  \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return MOE_EHIP; \
    } while (0)

size_t moe_route_workspace_bytes(int64_t T, int64_t d, int32_t E);
size_t moe_gemm_workspace_bytes(int32_t G);
moe_status_t moe_gemm_ksplit_f32(const void* x, const void* w, int64_t T, int64_t d, int32_t N, int32_t KS, float* C,
                                 hipStream_t s);

static inline bool moe_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// MOE_DEBUG builds (never the release library): the grouped GEMM's operand loads carry the
// operand's real extent in their buffer descriptors, so the hardware returns zeros for any
// load outside it instead of reading past the buffer, and the entry points copy the device
// index data they are given (group offsets, gather indices, expert ids) to the host and
// validate it before launching anything (a synchronising copy: not for graph capture).
#ifndef MOE_DEBUG
#define MOE_DEBUG 0
#endif
#if MOE_DEBUG
#include <vector>
static inline bool moe_debug_fetch_i32(const int32_t* dev, int64_t n, hipStream_t s, std::vector<int32_t>& out) {
    out.assign((size_t)(n > 0 ? n : 0), 0);
    if (n <= 0) return true;
    if (hipMemcpyAsync(out.data(), dev, (size_t)n * 4, hipMemcpyDeviceToHost, s) != hipSuccess) return false;
    return hipStreamSynchronize(s) == hipSuccess;
}
#endif

// One rounding of an exact product, shared by the combine's transpose and the quantiser's
// scaled-gather mode so both form the same bits. The product of two fp32 values is exact in
// fp64; rounding it to fp32 with round-to-odd (truncate, then set the last bit if anything
// was cut off) and then once more to bf16 gives the bf16 nearest the exact product, since
// fp32 carries more than bf16's precision plus two bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ float mul_round_odd(float w, float x) {
    const double p = (double)w * (double)x;
    float f = (float)p;
    if ((double)f != p) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(p)) u -= 1;   // truncate toward zero ...
        f = __uint_as_float(u | 1u);             // ... and mark inexact in the last bit
    }
    return f;
}

}  // namespace moe

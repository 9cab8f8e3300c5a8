// The SwiGLU derivative, shared by moe_swiglu_backward and the quantiser's fused SwiGLU-
// backward mode so both evaluate the same fp32 expression. With h = silu(g) * u and
// s = 1 / (1 + exp(-g)) (silu(g) = g s, its derivative s (1 + g (1 - s))):
//   dg = dh * u * s * (1 + g * (1 - s)),   du = dh * g * s
// ([Blog] Figure 3 paragraph: the experts are SwiGLU MLPs.)
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

__device__ __forceinline__ void swiglu_grad(float dh, float g, float u, float& dg, float& du) {
    const float sg = 1.f / (1.f + expf(-g));
    du = dh * (g * sg);
    dg = dh * u * (sg * (1.f + g * (1.f - sg)));
}

}  // namespace moe

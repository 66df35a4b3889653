// ssm_common.h -- device helpers shared by the selective-scan kernels (ssm_scan.hip and
// ssm_chunk.hip), so that every pass takes a token's step from the same arithmetic.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// The step of a token and head: softplus(dt) = log(1 + e^dt), or the raw dt.  Computed with
// the hardware exp and log: below dt = -4 (e^dt < 0.019) as the series e - e^2/2 + e^3/3 -
// e^4/4 (truncation below 2e-8 relative), elsewhere as log(1 + e^dt), whose argument is then
// at least 1.018 so the rounding of 1 + e^dt costs at most ~3e-6 relative; above 20 it is dt.
// Both directions use this one function, so the backward's replay gives the forward's bits.
__device__ __forceinline__ float ssm_step(float z, int softplus) {
    if (!softplus) return z;
    const float e = __expf(z);
    const float series = e * (1.f - e * (0.5f - e * (1.f / 3.f - e * 0.25f)));
    const float direct = __logf(1.f + e);
    return z > 20.f ? z : (z < -4.f ? series : direct);
}

}  // namespace gdn

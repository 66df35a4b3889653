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

// Buffer loads: a wave-uniform base (scalar registers), a per-lane byte offset and a scalar byte
// offset, so a block's or chunk's loads need no 64-bit vector address arithmetic.  Bases are
// taken at the block's or chunk's first token; the offsets used stay below 2^31.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const float *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ float bld(Rsrc r, uint32_t vbytes, uint32_t sbytes) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vbytes, sbytes, 0));
}

}  // namespace gdn

// rn_probe.hip -- plain streaming passes used as the practical bandwidth
// ceiling next to the kernels' own figures (measurement only; nothing on the
// RMSNorm path calls it).
//
// One grid-stride pass over n 16-byte vectors: each vector i of the R source
// streams is loaded (non-temporal), the loads are combined with XOR, and the
// result is stored (non-temporal) to vector i of each of the W destination
// streams.  This moves the same bytes with the same read:write mix as an
// operation whose streams have equal size, with no other work, and so bounds
// what any kernel with that mix can reach on the part.
#include <hip/hip_runtime.h>

#include "../../include/rmsnorm_gfx950.h"
#include "rn_device.h"

namespace rn {

struct MixArgs {
    const u32x4* src[4];
    u32x4* dst[5];
};

template <int R, int W>
__global__ __launch_bounds__(256) void k_stream_mix(MixArgs m, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        u32x4 v = __builtin_nontemporal_load(m.src[0] + i);
#pragma unroll
        for (int r = 1; r < R; ++r) v ^= __builtin_nontemporal_load(m.src[r] + i);
#pragma unroll
        for (int w = 0; w < W; ++w) __builtin_nontemporal_store(v, m.dst[w] + i);
    }
}

} // namespace rn

extern "C" int rn_stream_mix(const void* const* src, int nsrc, void* const* dst, int ndst, int64_t n16, int grid,
                             void* stream)
{
    if (!src || !dst) return RN_ERR_NULL;
    const int code = nsrc * 10 + ndst;
    if (code != 11 && code != 21 && code != 31 && code != 22 && code != 45) return RN_ERR_SHAPE;
    if (n16 < 0 || grid < 1 || grid > 65536) return RN_ERR_SHAPE;
    rn::MixArgs m{};
    for (int k = 0; k < nsrc; ++k) {
        if (!src[k]) return RN_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(src[k]) % 16) return RN_ERR_ALIGN;
        m.src[k] = static_cast<const rn::u32x4*>(src[k]);
    }
    for (int k = 0; k < ndst; ++k) {
        if (!dst[k]) return RN_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(dst[k]) % 16) return RN_ERR_ALIGN;
        m.dst[k] = static_cast<rn::u32x4*>(dst[k]);
    }
    if (n16 == 0) return RN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const dim3 g((unsigned)grid), b(256);
    switch (code) {
    case 11: hipLaunchKernelGGL((rn::k_stream_mix<1, 1>), g, b, 0, s, m, n16); break;
    case 21: hipLaunchKernelGGL((rn::k_stream_mix<2, 1>), g, b, 0, s, m, n16); break;
    case 31: hipLaunchKernelGGL((rn::k_stream_mix<3, 1>), g, b, 0, s, m, n16); break;
    case 22: hipLaunchKernelGGL((rn::k_stream_mix<2, 2>), g, b, 0, s, m, n16); break;
    default: hipLaunchKernelGGL((rn::k_stream_mix<4, 5>), g, b, 0, s, m, n16); break;
    }
    return hipGetLastError() == hipSuccess ? RN_OK : RN_ERR_LAUNCH;
}

// stream_probe.hip -- plain streaming passes for gfx950, the practical
// bandwidth ceiling next to the RMSNorm kernels' figures (measurement only).
// See stream_probe.h for the interface.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Streams {
    const u32x4* src[4];
    u32x4* dst[5];
};

// Work-groups are dispatched round-robin over the 8 XCDs (b % 8); give each
// XCD a contiguous run of logical indices.  Bijective for any grid.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t G)
{
    const int64_t q = G / 8, r = G % 8, x = b % 8, i = b / 8;
    return x * q + (x < r ? x : r) + i;
}

template <int R, int W, int VPT>
__device__ __forceinline__ void tile(const Streams& m, int64_t base, int64_t n, int wgs, uint32_t& acc)
{
    u32x4 v[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int64_t i = base + (int64_t)k * wgs;
        const int64_t c = i < n ? i : n - 1;             // clamped, always in bounds
        if constexpr (R > 0) {
            v[k] = __builtin_nontemporal_load(m.src[0] + c);
#pragma unroll
            for (int r = 1; r < R; ++r) v[k] ^= __builtin_nontemporal_load(m.src[r] + c);
        } else {
            const uint32_t lo = (uint32_t)i;
            v[k] = u32x4{lo, ~lo, lo, ~lo};
        }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int64_t i = base + (int64_t)k * wgs;
        if constexpr (W > 0) {
            if (i < n) {
#pragma unroll
                for (int w = 0; w < W; ++w) __builtin_nontemporal_store(v[k], m.dst[w] + i);
            }
        } else {
            if (i < n) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
        }
    }
}

template <int R, int W, int VPT>
__global__ __launch_bounds__(1024) void k_mix(Streams m, int64_t n, int order, uint32_t* sink)
{
    const int wgs = blockDim.x;
    const int64_t G = gridDim.x;
    const int64_t T = (int64_t)wgs * VPT;               // vectors per tile
    uint32_t acc = 0;
    if (order == 2) {
        const int64_t ntiles = (n + T - 1) / T;
        const int64_t b = blockIdx.x;
        const int64_t lo = ntiles * b / G, hi = ntiles * (b + 1) / G;
        for (int64_t t = lo; t < hi; ++t) tile<R, W, VPT>(m, t * T + threadIdx.x, n, wgs, acc);
    } else {
        const int64_t L = order == 1 ? xcd_order(blockIdx.x, G) : (int64_t)blockIdx.x;
        for (int64_t base = L * T + threadIdx.x; base - threadIdx.x < n; base += G * T)
            tile<R, W, VPT>(m, base, n, wgs, acc);
    }
    if constexpr (W == 0) {
        if (acc == 0x9E3779B9u) sink[0] = acc;
    }
}

template <int R, int W>
hipError_t go(const Streams& m, int64_t n, int grid, int wgs, int vpt, int order, uint32_t* sink, hipStream_t s)
{
    const dim3 g((unsigned)grid), b((unsigned)wgs);
    switch (vpt) {
    case 1: hipLaunchKernelGGL((k_mix<R, W, 1>), g, b, 0, s, m, n, order, sink); break;
    case 2: hipLaunchKernelGGL((k_mix<R, W, 2>), g, b, 0, s, m, n, order, sink); break;
    case 4: hipLaunchKernelGGL((k_mix<R, W, 4>), g, b, 0, s, m, n, order, sink); break;
    default: hipLaunchKernelGGL((k_mix<R, W, 8>), g, b, 0, s, m, n, order, sink); break;
    }
    return hipGetLastError();
}

template <int R>
hipError_t go_w(int ndst, const Streams& m, int64_t n, int grid, int wgs, int vpt, int order, uint32_t* sink,
                hipStream_t s)
{
    switch (ndst) {
    case 0: if constexpr (R > 0) return go<R, 0>(m, n, grid, wgs, vpt, order, sink, s); else return hipErrorInvalidValue;
    case 1: return go<R, 1>(m, n, grid, wgs, vpt, order, sink, s);
    case 2: return go<R, 2>(m, n, grid, wgs, vpt, order, sink, s);
    case 3: return go<R, 3>(m, n, grid, wgs, vpt, order, sink, s);
    case 4: return go<R, 4>(m, n, grid, wgs, vpt, order, sink, s);
    default: return go<R, 5>(m, n, grid, wgs, vpt, order, sink, s);
    }
}

} // namespace

extern "C" int sp_stream_mix(const void* const* src, int nsrc, void* const* dst, int ndst, int64_t n16, int grid,
                             int wgs, int vpt, int order, uint32_t* sink, void* stream)
{
    if (nsrc < 0 || nsrc > 4 || ndst < 0 || ndst > 5 || nsrc + ndst == 0) return 2;
    if (n16 < 0 || grid < 1 || grid > 65536) return 2;
    if (wgs != 64 && wgs != 128 && wgs != 256 && wgs != 512 && wgs != 1024) return 2;
    if (vpt != 1 && vpt != 2 && vpt != 4 && vpt != 8) return 2;
    if (order < 0 || order > 2) return 2;
    if ((nsrc > 0 && !src) || (ndst > 0 && !dst)) return 1;
    if (ndst == 0 && !sink) return 1;
    Streams m{};
    for (int k = 0; k < nsrc; ++k) {
        if (!src[k]) return 1;
        if (reinterpret_cast<uintptr_t>(src[k]) % 16) return 4;
        m.src[k] = static_cast<const u32x4*>(src[k]);
    }
    for (int k = 0; k < ndst; ++k) {
        if (!dst[k]) return 1;
        if (reinterpret_cast<uintptr_t>(dst[k]) % 16) return 4;
        m.dst[k] = static_cast<u32x4*>(dst[k]);
    }
    if (ndst == 0 && reinterpret_cast<uintptr_t>(sink) % 4) return 4;
    if (n16 == 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e;
    switch (nsrc) {
    case 0: e = go_w<0>(ndst, m, n16, grid, wgs, vpt, order, sink, s); break;
    case 1: e = go_w<1>(ndst, m, n16, grid, wgs, vpt, order, sink, s); break;
    case 2: e = go_w<2>(ndst, m, n16, grid, wgs, vpt, order, sink, s); break;
    case 3: e = go_w<3>(ndst, m, n16, grid, wgs, vpt, order, sink, s); break;
    default: e = go_w<4>(ndst, m, n16, grid, wgs, vpt, order, sink, s); break;
    }
    return e == hipSuccess ? 0 : 9;
}

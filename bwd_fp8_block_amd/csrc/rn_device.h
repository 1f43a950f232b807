// rn_device.h -- gfx950 device helpers shared by the RMSNorm kernels.
//
// Rows are processed in 16-byte vectors ("chunks"): 8 bf16 or 4 fp32 values.
// A row is owned by a group of LPR consecutive lanes (16, 32, 64, or a
// multiple of 64 spanning several wavefronts); lane l of the group owns
// chunks l, l + LPR, l + 2*LPR, ... so that every load instruction of a
// wavefront covers 64 * 16 = 1 KiB of contiguous row memory.
//
// Reductions inside a group use DPP lane permutations (quad_perm, half-row
// and row mirrors) within each 16-lane DPP row, one ds_swizzle across the two
// 16-lane halves of 32 lanes, and readlane across the two 32-lane halves of a
// wavefront.  Every lane of the group ends with the same value, and the
// combination order is fixed, so results are reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Elements per 16-byte chunk for a storage dtype.
template <int DT> struct Elems { static constexpr int value = (DT == DT_F32) ? 4 : 8; };

// ---------------------------------------------------------------------------
// Global memory access.  NT selects non-temporal (streaming) hints.
// ---------------------------------------------------------------------------
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NT>
__device__ __forceinline__ void st8(u32x2* p, u32x2 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Make a register value opaque to the optimizer for one use site, so that a
// loop-invariant packed value is not unpacked once and kept live in its wider
// form across the loop (which would cost registers, not time).
__device__ __forceinline__ void opaque(u32x4& v) { asm volatile("" : "+v"(v)); }

// Materialise a value in its register at this point of the program: keeps the
// compiler from sinking the arithmetic that produced it past later work (and
// holding that work's inputs live in the meantime).
__device__ __forceinline__ void settle(double& v) { asm volatile("" : "+v"(v)); }

// A value that is the same in every lane of the wavefront, made visible as
// such to the compiler (it then lives in scalar registers, and addresses built
// from it use scalar arithmetic).  Only for values that really are uniform: the
// first active lane's value is taken.
__device__ __forceinline__ int64_t wave_uniform(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Zero a loaded vector when its chunk or row is out of range (the load itself
// was issued from a clamped, always valid address).
__device__ __forceinline__ u32x4 keep_if(bool ok, const u32x4& v)
{
    return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A bf16 value is the upper half of a binary32, so unpacking
// is a shift or a mask; packing uses v_cvt_pk_bf16_f32 (round to nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// fp16 <-> fp32 (IEEE binary16; conversion to fp16 rounds to nearest even).
__device__ __forceinline__ float f16lo(uint32_t u) { return (float)__builtin_bit_cast(f16x2, u)[0]; }
__device__ __forceinline__ float f16hi(uint32_t u) { return (float)__builtin_bit_cast(f16x2, u)[1]; }

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    f16x2 h = __builtin_convertvector(v, f16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// 16-bit storage types by dtype: low / high half of a word, and packing.
template <int DT> __device__ __forceinline__ float lo16(uint32_t u) { return DT == DT_F16 ? f16lo(u) : bf16lo(u); }
template <int DT> __device__ __forceinline__ float hi16(uint32_t u) { return DT == DT_F16 ? f16hi(u) : bf16hi(u); }
template <int DT> __device__ __forceinline__ uint32_t pack16x2(float lo, float hi)
{
    return DT == DT_F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// Unpack one chunk of storage dtype DT into E fp32 values.
template <int DT>
__device__ __forceinline__ void unpack(const u32x4& v, float* f)
{
    if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = bf16lo(v[k]);
            f[2 * k + 1] = bf16hi(v[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
    }
}

// Pack E fp32 values into one chunk of storage dtype DT (RNE for bf16).
template <int DT>
__device__ __forceinline__ u32x4 pack(const float* f)
{
    u32x4 v;
    if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(f[k]);
    }
    return v;
}

// ---------------------------------------------------------------------------
// Lane permutations.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// DPP controls used below.
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <- lane 15-i within 16
constexpr int SWZ_XOR16 = 0x401F;      // ds_swizzle bit mode: lane ^ 16 within 32

__device__ __forceinline__ float swz_xor16(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SWZ_XOR16));
}

__device__ __forceinline__ float readlane_f32(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of LPRC lanes (LPRC in {4, 8, 16, 32, 64}); every
// lane of a group receives the same sum.  Must run with all 64 lanes active.
template <int LPRC>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(LPRC == 4 || LPRC == 8 || LPRC == 16 || LPRC == 32 || LPRC == 64, "group width");
    v += dpp_f32<DPP_QUAD_XOR1>(v);
    v += dpp_f32<DPP_QUAD_XOR2>(v);
    if constexpr (LPRC >= 8) v += dpp_f32<DPP_HALF_MIRROR>(v);
    if constexpr (LPRC >= 16) v += dpp_f32<DPP_ROW_MIRROR>(v);
    if constexpr (LPRC >= 32) v += swz_xor16(v);
    if constexpr (LPRC >= 64) v = readlane_f32(v, 0) + readlane_f32(v, 32);
    return v;
}

// Row-group geometry of a work-group.  LPRC is the compile-time class of the
// group width: 4 .. 32 (several rows per wavefront) or 64, meaning the group
// is lpr = 64 * wpr lanes wide (wpr whole wavefronts, wpr chosen at launch).
template <int LPRC>
struct Rows {
    int lpr;    // lanes per row group
    int gpw;    // row groups per work-group
    int wpr;    // wavefronts per row group (1 when LPRC < 64)
    int grp;    // this thread's row group
    int lane;   // this thread's lane inside its row group

    __device__ __forceinline__ Rows(int lpr_rt)
    {
        lpr = (LPRC < 64) ? LPRC : lpr_rt;
        gpw = blockDim.x / lpr;
        wpr = (LPRC < 64) ? 1 : lpr >> 6;
        grp = threadIdx.x / lpr;
        lane = threadIdx.x - grp * lpr;
    }

    // Sum of v over the row group, the same in every lane.  When the group
    // spans several wavefronts the per-wavefront sums meet in LDS (slot
    // `red`, two buffers alternating with the iteration parity `it`) and are
    // added in wavefront order.  Must be reached by every thread of the
    // work-group (it contains a barrier when wpr > 1).
    __device__ __forceinline__ float sum(float v, float (*red)[16], int it) const
    {
        v = group_sum<LPRC>(v);
        if constexpr (LPRC == 64) {
            if (wpr > 1) {
                if ((threadIdx.x & 63) == 0) red[it & 1][threadIdx.x >> 6] = v;
                __syncthreads();
                float t = 0.0f;
                for (int k = 0; k < wpr; ++k) t += red[it & 1][grp * wpr + k];
                v = t;
            }
        }
        return v;
    }
};

// Unsigned max over aligned groups of 16 lanes (one DPP row).
__device__ __forceinline__ uint32_t max16_u32(uint32_t v)
{
    v = max(v, dpp_u32<DPP_QUAD_XOR1>(v));
    v = max(v, dpp_u32<DPP_QUAD_XOR2>(v));
    v = max(v, dpp_u32<DPP_HALF_MIRROR>(v));
    v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));
    return v;
}

// Software pipeline over the rows of a row group: PD row buffers in a ring,
// PD-1 rows of loads in flight while one row is processed.  load(buf, it)
// issues the loads of iteration `it`; process(buf, it) consumes them.  All
// buffer indices are compile-time constants after unrolling; the branches
// depend only on n_it, which is uniform across the work-group, so `process`
// may contain barriers.
//
// Two forms, which differ in where the compiler places its waits on the
// vector-memory counter (computed per control-flow merge on gfx9):
//   STEADY   whole blocks of PD iterations issue every prefetch
//            unconditionally (iterations past n_it load the walk's clamped
//            row, a real row, and are never processed); the last fewer than
//            PD iterations follow without new loads.  Each row then waits
//            only for its own loads: PD-1 rows stay in flight.
//   guarded  a prefetch is issued only for a row that exists.  The merge
//            after the guarded load makes the compiler's wait for the current
//            row a drain of the prefetch and of earlier stores as well, so
//            memory traffic advances about one row per row group at a time.
// Which form streams faster depends on the kernel's mix of reads and writes
// and on how many row groups share a CU; each kernel picks the one measured
// faster on MI355X.
template <int PD, bool STEADY, class Buf, class LoadF, class ProcF>
__device__ __forceinline__ void row_pipeline(int n_it, LoadF&& load, ProcF&& process)
{
    Buf b[PD];
    if constexpr (STEADY) {
#pragma unroll
        for (int k = 0; k < PD - 1; ++k) load(b[k], k);
        int it = 0;
        for (; it + PD <= n_it; it += PD) {
#pragma unroll
            for (int k = 0; k < PD; ++k) {
                load(b[(k + PD - 1) % PD], it + k + PD - 1);
                process(b[k], it + k);
            }
        }
#pragma unroll
        for (int k = 0; k < PD - 1; ++k)
            if (it + k < n_it) process(b[k], it + k);
    } else {
#pragma unroll
        for (int k = 0; k < PD - 1; ++k)
            if (k < n_it) load(b[k], k);
        for (int it = 0; it < n_it; it += PD) {
#pragma unroll
            for (int k = 0; k < PD; ++k) {
                if (it + k < n_it) {
                    if (it + k + PD - 1 < n_it) load(b[(k + PD - 1) % PD], it + k + PD - 1);
                    process(b[k], it + k);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Work partition helpers.
// ---------------------------------------------------------------------------

// Work-groups are dispatched round-robin over the 8 XCDs of the MI355X
// (blockIdx.x % 8 selects the XCD).  Map them so that each XCD receives a
// contiguous run of logical row chunks: neighbouring chunks then share the
// XCD's L2, which merges the partial-line writes of per-row outputs (rstd,
// block scales) that straddle a chunk boundary.  Bijective for any grid size.
__device__ __forceinline__ int64_t xcd_chunk(int64_t b, int64_t G)
{
    const int64_t nx = 8;
    int64_t q = G / nx, r = G % nx;
    int64_t x = b % nx, i = b / nx;
    return x * q + (x < r ? x : r) + i;
}

// Rows [lo, hi) of chunk g out of G chunks over T rows (balanced, exact).
__device__ __forceinline__ void chunk_rows(int64_t g, int64_t G, int64_t T, int64_t& lo, int64_t& hi)
{
    lo = (g * T) / G;
    hi = ((g + 1) * T) / G;
}

// The rows a row group visits: row(it) = first + it * step for it < n_it;
// rows at or past `limit` are padding (their loads use the clamped row
// `last` = limit - 1, a real row since the grid never exceeds the row count
// and so no chunk ends at row 0; nothing is stored for padding rows).
//   contiguous:  work-group L owns the chunk [lo, hi) of rows; its gpw groups
//                interleave inside it (first = lo + grp, step = gpw).
//   interleaved: at iteration it the work-groups cover the rows
//                [it*G*gpw, (it+1)*G*gpw) together, so the GPU streams through
//                the tensor as one moving window; L is XCD-aware, so each
//                XCD's share of the window is contiguous.
struct RowWalk {
    int64_t first, step, limit, last;
    int n_it;
    __device__ __forceinline__ int64_t row(int it) const { return first + (int64_t)it * step; }
    __device__ __forceinline__ bool valid(int64_t r) const { return r < limit; }
    __device__ __forceinline__ int64_t clamp(int64_t r) const { return r < limit ? r : last; }
};

__device__ __forceinline__ RowWalk row_walk(bool interleaved, int64_t L, int64_t G, int64_t T, int gpw, int grp)
{
    RowWalk w;
    if (interleaved) {
        w.first = L * gpw + grp;
        w.step = G * gpw;
        w.limit = T;
        w.n_it = (int)((T - L * gpw + w.step - 1) / w.step);
    } else {
        int64_t lo, hi;
        chunk_rows(L, G, T, lo, hi);
        w.first = lo + grp;
        w.step = gpw;
        w.limit = hi;
        w.n_it = (int)((hi - lo + gpw - 1) / gpw);
    }
    w.last = w.limit > 0 ? w.limit - 1 : 0;
    return w;
}

} // namespace rn

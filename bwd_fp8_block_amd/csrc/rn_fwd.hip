// rn_fwd.hip -- RMSNorm forward for gfx950.
//
// Operation ([C] = FlashInfer commit #5741 "cake_rmsnorm_train", Summary and
// Design: Forward): per row an fp32 sum of squares, rstd = 1/sqrt(ss/H + eps)
// with IEEE square root and division, y = round(x * rstd * w), and the fp32
// rstd stored for the backward.
//
// Mapping: the grid is a set of row chunks (one per work-group, contiguous
// rows, XCD-aware order).  Inside a work-group, gpw row groups of lpr lanes
// each take every gpw-th row of the chunk.  A row stays in registers between
// the sum-of-squares pass and the write pass, so x is read from HBM once; w is
// read once per work-group and kept in registers.  The row reduction is a DPP
// butterfly inside the wavefront, plus one LDS exchange when a row spans
// several wavefronts.  With PF the next row's loads are issued before the
// current row is reduced, so each wavefront keeps two rows of loads in flight.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// Load the NV chunks of one row that this lane owns (zeros when masked off).
template <int NV, bool NT>
__device__ __forceinline__ void load_row(u32x4 (&v)[NV], const u32x4* row, int lane, int lpr, int nch, bool valid)
{
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + lpr * i;
        if (valid && c < nch) v[i] = ld16<NT>(row + c);
        else v[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int XT, int WT, int LPRC, int NV, int WGMAX, bool PF, bool NTL, bool NTS>
__global__ __launch_bounds__(WGMAX) void k_rmsnorm_fwd(FwdArgs a)
{
    constexpr int E = Elems<XT>::value;
    constexpr int WPER = (WT == DT_F32) ? 4 : 8;    // w values per 16-byte word
    constexpr int WCH = E / WPER;                   // w words per x chunk
    constexpr int XB = (XT == DT_BF16) ? 2 : 4;     // bytes per x element

    __shared__ float red[2][16];

    const Rows<LPRC> R(a.lpr);
    const int lane = R.lane, lpr = R.lpr, gpw = R.gpw;
    const int nch = a.nch;

    int64_t lo, hi;
    chunk_rows(xcd_chunk(blockIdx.x, gridDim.x), gridDim.x, a.T, lo, hi);
    const int n_it = (int)((hi - lo + gpw - 1) / gpw);

    // w for this lane's chunks, raw words kept in registers.
    u32x4 wr[NV][WCH];
    {
        const u32x4* wp = static_cast<const u32x4*>(a.w);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + lpr * i;
#pragma unroll
            for (int k = 0; k < WCH; ++k) wr[i][k] = (c < nch) ? wp[c * WCH + k] : u32x4{0u, 0u, 0u, 0u};
        }
    }

    const char* xbase = static_cast<const char*>(a.x);
    char* ybase = static_cast<char*>(a.y);

    u32x4 nxt[NV];
    if constexpr (PF) {
        const int64_t r0 = lo + R.grp;
        load_row<NV, NTL>(nxt, reinterpret_cast<const u32x4*>(xbase + r0 * a.ldx * XB), lane, lpr, nch, r0 < hi);
    }

    for (int it = 0; it < n_it; ++it) {
        const int64_t r = lo + R.grp + (int64_t)it * gpw;
        const bool valid = r < hi;
        u32x4 xv[NV];
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < NV; ++i) xv[i] = nxt[i];
            const int64_t rn = r + gpw;
            if (it + 1 < n_it)
                load_row<NV, NTL>(nxt, reinterpret_cast<const u32x4*>(xbase + rn * a.ldx * XB), lane, lpr, nch, rn < hi);
        } else {
            load_row<NV, NTL>(xv, reinterpret_cast<const u32x4*>(xbase + r * a.ldx * XB), lane, lpr, nch, valid);
        }

        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float f[E];
            unpack<XT>(xv[i], f);
#pragma unroll
            for (int e = 0; e < E; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
        }
        ss = R.sum(ss, red, it);

        const float ms = ss / (float)a.H;
        const float rs = 1.0f / __builtin_sqrtf(ms + a.eps);

        u32x4* yrow = reinterpret_cast<u32x4*>(ybase + r * a.ldy * XB);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + lpr * i;
            float f[E], wf[E], o[E];
            unpack<XT>(xv[i], f);
#pragma unroll
            for (int k = 0; k < WCH; ++k) unpack<WT>(wr[i][k], wf + k * WPER);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = (f[e] * rs) * wf[e];
            if (valid && c < nch) st16<NTS>(yrow + c, pack<XT>(o));
        }
        if (valid && lane == 0) a.rstd[r] = rs;
    }
}

// ---------------------------------------------------------------------------
// Variant table and dispatch: template on the group class (16, 32, 64+) and
// on the vectors per lane; the group width for class 64 is a launch argument.
// ---------------------------------------------------------------------------
constexpr bool FWD_PF = true;
constexpr bool FWD_NTL = false;
constexpr bool FWD_NTS = false;

template <int XT, int WT, int LPRC, int NV, int WGMAX>
static hipError_t fwd_go(const FwdArgs& a, const Policy& p, hipStream_t s)
{
    hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, FWD_PF, FWD_NTL, FWD_NTS>),
                       dim3((unsigned)p.grid), dim3(p.wgs), 0, s, a);
    return hipGetLastError();
}

// (group class, vectors per lane, largest work-group) triples compiled.
#define RN_FWD_VARIANTS(X) X(16, 1, 256) X(16, 2, 256) X(16, 4, 256) X(32, 2, 256) X(32, 4, 256)         \
    X(64, 1, 256) X(64, 2, 256) X(64, 3, 256) X(64, 4, 256) X(64, 5, 256) X(64, 6, 256) X(64, 7, 256) \
    X(64, 8, 256) X(64, 8, 512)

bool fwd_variant_exists(int lprc, int nv, int wgs)
{
#define X(C, N, W) if (lprc == C && nv == N && wgs <= W) return true;
    RN_FWD_VARIANTS(X)
#undef X
    return false;
}

template <int XT, int WT>
static hipError_t fwd_dispatch(const FwdArgs& a, const Policy& p, hipStream_t s)
{
    const int lprc = p.lpr < 64 ? p.lpr : 64;
#define X(C, N, W) if (lprc == C && p.nv == N && p.wgs <= W) return fwd_go<XT, WT, C, N, W>(a, p, s);
    RN_FWD_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int x_dtype, int w_dtype, const Policy& p, hipStream_t s)
{
    if (x_dtype == DT_BF16 && w_dtype == DT_BF16) return fwd_dispatch<DT_BF16, DT_BF16>(a, p, s);
    if (x_dtype == DT_BF16 && w_dtype == DT_F32) return fwd_dispatch<DT_BF16, DT_F32>(a, p, s);
    if (x_dtype == DT_F32 && w_dtype == DT_F32) return fwd_dispatch<DT_F32, DT_F32>(a, p, s);
    return hipErrorInvalidValue;
}

} // namespace rn

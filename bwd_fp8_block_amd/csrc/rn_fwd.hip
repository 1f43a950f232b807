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
// several wavefronts.  Two row buffers alternate, so each wavefront keeps the
// next row's loads in flight while it reduces and writes the current one.
// Loads are never predicated: out-of-range chunks and rows load from a
// clamped in-bounds address and are zeroed, which keeps the loads in one
// unbranched batch.  NT selects non-temporal (streaming) loads and stores.
//
// Forms (MODE):
//   FWD_PLAIN     rows r = 0 .. T-1 at x + r*ldx.
//   FWD_RESIDUAL  ([C] API and Design: Forward, the training forward with a
//                 residual): the row read is h_new = x + u, added in fp32 and
//                 rounded once to x's dtype, stored, and normalised in place
//                 of x.
//   FWD_HEADS     per-head RMSNorm ([Q] = FlashInfer PR #6332, QKV projection
//                 + QK-RMSNorm + RoPE overlapped with the Ulysses head exchange,
//                 Description, operator math): row r = t*heads + h is the
//                 head_dim slice at x + t*ldx + h*ldxh, with the shared
//                 head_dim weight; rstd[r] is optional.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

template <int XT, int WT, int LPRC, int NV, int WGMAX, bool NT, int PD, int MODE>
__global__ __launch_bounds__(WGMAX) void k_rmsnorm_fwd(FwdArgs a)
{
    constexpr bool RES = MODE == FWD_RESIDUAL;
    constexpr bool HEADS = MODE == FWD_HEADS;
    constexpr int E = Elems<XT>::value;
    constexpr int WPER = (WT == DT_F32) ? 4 : 8;    // w values per 16-byte word
    constexpr int WCH = E / WPER;                   // w words per x chunk
    constexpr int XB = (XT == DT_BF16) ? 2 : 4;     // bytes per x element

    __shared__ float red[2][16];

    const Rows<LPRC> R(a.lpr);
    const int lane = R.lane, lpr = R.lpr, gpw = R.gpw;
    const int nch = a.nch;

    const RowWalk W = row_walk(a.interleave != 0, xcd_chunk(blockIdx.x, gridDim.x), gridDim.x, a.T, gpw, R.grp);

    // This lane's chunks: index (clamped into the row so that every load is
    // in bounds) and whether it is real.
    int cix[NV];
    bool cok[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + lpr * i;
        cok[i] = c < nch;
        cix[i] = cok[i] ? c : nch - 1;
    }

    // w for this lane's chunks, raw (packed) words kept in registers.
    u32x4 wr[NV][WCH];
    {
        const u32x4* wp = static_cast<const u32x4*>(a.w);
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int k = 0; k < WCH; ++k) wr[i][k] = keep_if(cok[i], wp[cix[i] * WCH + k]);
    }

    const char* xbase = static_cast<const char*>(a.x);
    const char* ubase = static_cast<const char*>(a.u);
    char* ybase = static_cast<char*>(a.y);
    char* hbase = static_cast<char*>(a.h);

    // Per-head rows: the token of row r is floor(r / heads), taken as a
    // multiply and a shift by the host's constants (division by an invariant
    // integer, Granlund and Montgomery 1994): with l = ceil(log2 heads) and
    // m = ceil(2^(31+l) / heads) < 2^32, floor(r * m / 2^(31+l)) equals
    // floor(r / heads) for every r < 2^31 (rows < 2^31 is a host check).
    auto token_of = [&](uint32_t rr) -> uint32_t {
        return (uint32_t)(((uint64_t)rr * a.hmul) >> a.hshift);
    };
    // Element offsets of row r in x and in y (u and h_new use plain strides).
    auto xoff = [&](int64_t r) -> int64_t {
        if constexpr (HEADS) {
            const uint32_t rr = (uint32_t)r, t = token_of(rr);
            return (int64_t)t * a.ldx + (int64_t)(rr - t * (uint32_t)a.heads) * a.ldxh;
        } else {
            return r * a.ldx;
        }
    };
    auto yoff = [&](int64_t r) -> int64_t {
        if constexpr (HEADS) {
            const uint32_t rr = (uint32_t)r, t = token_of(rr);
            return (int64_t)t * a.ldy + (int64_t)(rr - t * (uint32_t)a.heads) * a.ldyh;
        } else {
            return r * a.ldy;
        }
    };

    // Rows past the end of the walk load from a clamped in-bounds row and
    // store nothing.  Loaded registers are not touched until they are used,
    // so the next row's loads stay in flight while this row is processed.
    struct RowBuf {
        u32x4 v[NV];
        u32x4 u[RES ? NV : 1];
    };
    auto load = [&](RowBuf& b, int it) {
        const int64_t rr = W.clamp(W.row(it));
        const u32x4* row = reinterpret_cast<const u32x4*>(xbase + xoff(rr) * XB);
#pragma unroll
        for (int i = 0; i < NV; ++i) b.v[i] = ld16<NT>(row + cix[i]);
        if constexpr (RES) {
            const u32x4* urow = reinterpret_cast<const u32x4*>(ubase + rr * a.ldu * XB);
#pragma unroll
            for (int i = 0; i < NV; ++i) b.u[i] = ld16<NT>(urow + cix[i]);
        }
    };

    auto process = [&](const RowBuf& b, int it) {
        // The row that is normalised: x, or h_new = round(x + u).
        u32x4 xv[NV];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (RES) {
                float f[E], g[E];
                unpack<XT>(b.v[i], f);
                unpack<XT>(b.u[i], g);
#pragma unroll
                for (int e = 0; e < E; ++e) f[e] += g[e];
                xv[i] = pack<XT>(f);
            } else {
                xv[i] = b.v[i];
            }
            float f[E];
            unpack<XT>(keep_if(cok[i], xv[i]), f);      // clamped duplicate chunks add nothing
#pragma unroll
            for (int e = 0; e < E; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
        }
        ss = R.sum(ss, red, it);
        const int64_t r = W.row(it);
        const float ms = ss / (float)a.H;
        const float rs = 1.0f / __builtin_sqrtf(ms + a.eps);
        if (W.valid(r)) {
            u32x4* yrow = reinterpret_cast<u32x4*>(ybase + yoff(r) * XB);
            if constexpr (RES) {
                u32x4* hrow = reinterpret_cast<u32x4*>(hbase + r * a.ldh * XB);
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (cok[i]) st16<NT>(hrow + cix[i], xv[i]);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float f[E], wf[E], o[E];
                u32x4 xc = xv[i];
                opaque(xc);               // unpack again rather than keep E floats live
                unpack<XT>(xc, f);
#pragma unroll
                for (int q = 0; q < WCH; ++q) {
                    if constexpr (LPRC == 64 || NV * E > 32) opaque(wr[i][q]);   // short rows: w stays unpacked
                    unpack<WT>(wr[i][q], wf + q * WPER);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = (f[e] * rs) * wf[e];
                if (cok[i]) st16<NT>(yrow + cix[i], pack<XT>(o));
            }
            if (lane == 0 && (!HEADS || a.rstd)) a.rstd[r] = rs;
        }
    };

    // PD row buffers in a ring: the next PD-1 rows' loads are in flight while
    // the current row is reduced and written.
    row_pipeline<PD, false, RowBuf>(W.n_it, load, process);
}

// ---------------------------------------------------------------------------
// Variant table and dispatch: template on the group class (16, 32, 64+) and
// on the vectors per lane; the group width for class 64 is a launch argument.
// ---------------------------------------------------------------------------
template <int XT, int WT, int LPRC, int NV, int WGMAX, int MODE>
static hipError_t fwd_go(const FwdArgs& a, const Policy& p, hipStream_t s)
{
    const dim3 g((unsigned)p.grid), b(p.wgs);
    if constexpr (MODE == FWD_HEADS) {
        // per-head rows are short (head_dim <= 128 vectors): sub-wave groups,
        // streaming accesses, two row buffers
        if constexpr (LPRC < 64 && NV <= 4) {
            hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, true, 2, MODE>), g, b, 0, s, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        // The residual form is compiled with streaming accesses only.
        constexpr bool RES = MODE == FWD_RESIDUAL;
        const bool nt = RES || (p.flags & RN_FLAG_NT) != 0;
        if constexpr (NV <= 4) {
            // short per-lane rows: a third row buffer is affordable
            if (((p.flags >> 4) & 7) == 3) {
                if (nt) hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, true, 3, MODE>), g, b, 0, s, a);
                else if constexpr (!RES) hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, false, 3, MODE>), g, b, 0, s, a);
                return hipGetLastError();
            }
        }
        if (nt) hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, true, 2, MODE>), g, b, 0, s, a);
        else if constexpr (!RES) hipLaunchKernelGGL((k_rmsnorm_fwd<XT, WT, LPRC, NV, WGMAX, false, 2, MODE>), g, b, 0, s, a);
        return hipGetLastError();
    }
}

// (group class, vectors per lane, largest work-group) triples compiled.
#define RN_FWD_VARIANTS(X) X(4, 4, 256) X(8, 1, 256) X(8, 2, 256) X(8, 4, 256)                            \
    X(16, 1, 256) X(16, 2, 256) X(16, 4, 256) X(32, 2, 256) X(32, 4, 256)                                \
    X(64, 1, 256) X(64, 2, 256) X(64, 3, 256) X(64, 4, 256) X(64, 5, 256) X(64, 6, 256) X(64, 7, 256) \
    X(64, 8, 256) X(64, 5, 512) X(64, 6, 512) X(64, 7, 512) X(64, 8, 512)

bool fwd_variant_exists(int lprc, int nv, int wgs)
{
#define X(C, N, W) if (lprc == C && nv == N && wgs <= W) return true;
    RN_FWD_VARIANTS(X)
#undef X
    return false;
}

template <int XT, int WT, int MODE>
static hipError_t fwd_dispatch(const FwdArgs& a, const Policy& p, hipStream_t s)
{
    const int lprc = p.lpr < 64 ? p.lpr : 64;
#define X(C, N, W) if (lprc == C && p.nv == N && p.wgs <= W) return fwd_go<XT, WT, C, N, W, MODE>(a, p, s);
    RN_FWD_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t fwd_dtypes(const FwdArgs& a, int x_dtype, int w_dtype, const Policy& p, hipStream_t s)
{
    if (x_dtype == DT_BF16 && w_dtype == DT_BF16) return fwd_dispatch<DT_BF16, DT_BF16, MODE>(a, p, s);
    if (x_dtype == DT_BF16 && w_dtype == DT_F32) return fwd_dispatch<DT_BF16, DT_F32, MODE>(a, p, s);
    if (x_dtype == DT_F32 && w_dtype == DT_F32) return fwd_dispatch<DT_F32, DT_F32, MODE>(a, p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int x_dtype, int w_dtype, int mode, const Policy& p, hipStream_t s)
{
    switch (mode) {
    case FWD_PLAIN: return fwd_dtypes<FWD_PLAIN>(a, x_dtype, w_dtype, p, s);
    case FWD_RESIDUAL: return fwd_dtypes<FWD_RESIDUAL>(a, x_dtype, w_dtype, p, s);
    case FWD_HEADS: return fwd_dtypes<FWD_HEADS>(a, x_dtype, w_dtype, p, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace rn

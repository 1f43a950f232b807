// rn_bwd.hip -- RMSNorm backward (dx and dw in one pass over the rows) for gfx950.
//
// Operation ([C] = FlashInfer commit #5741 "cake_rmsnorm_train", Design:
// Backward and Determinism; [L] = Liger-Kernel PR #1336, the fused single-pass
// dX+dW strip-reduction backward):
//   xhat = x * rstd;  c = mean_j(g * w * xhat);  dx = rstd * (g*w - c*xhat)
//   dw_j = sum over rows of g * x * rstd
//
// Mapping.  The rows are split into G strips, one per work-group: a strip is
// either a contiguous chunk of rows or, in the interleaved walk used for
// streaming, every G-th block of GPW rows (all strips then move through the
// tensor as one window).  A work-group holds GPW row groups of LPR lanes,
// one row per group at a time.  Per row: 16-byte loads of g and x,
// fp32 dot product reduced across the row group (DPP, then LDS when a row
// spans several wavefronts), dx written back, and the dw contribution of the
// row added to per-lane FP64 accumulators for the lane's columns.
//
// dw accuracy.  For bf16 inputs g*x is exact in fp32 (8 + 8 significant
// bits), and (g*x)*rstd is exact in FP64 (16 + 24 bits), so each contribution
// enters the FP64 accumulator exactly; the only roundings of a strip partial
// are FP64 additions and the final fp32 rounding.  On the pages' hardware
// the same budget (every element within 1e-4 + 1e-4*|ref| of an FP64 sum,
// miles-ext-kernels PR #15, Summary) is met with compensated fp32 sums; on
// gfx950 FP64 FMA issues at the same rate as fp32 FMA, so plain FP64
// accumulation is the cheaper way to the same end.
//
// Each strip writes its fp32 partial row to the workspace, and a second
// kernel sums the G partials of every column in a fixed order in FP64 (no
// atomics: the result depends only on T, H and G, and is bitwise repeatable).
// When one strip walks all the rows (a few rows), its partial is dw itself
// and is written there directly: one launch, no workspace.  Adding the strip
// partials with fp32 atomics instead was measured over the per-element dw
// budget at T = 65536, H = 5120 (1.03x), and was not faster than this second
// kernel, so both modes of the entry point use this path.  A single launch
// would need the strips to wait for the last one before the column sums can
// start (every partial is complete only at the end of its strip), that is a
// grid-wide barrier; it is not used.
//
// Residual form (RES; [C] API and Design: Backward, the training backward
// with a residual): the gradient arriving along the residual stream is added
// to dx in fp32 before the one rounding into x's dtype; dw is unchanged.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// Workspace layout: column blocks of RN_PART_COLS = 16 columns; block b holds
// the G strip partials of its columns contiguously, [b][strip][column % 16],
// so that the reduce reads each block as one contiguous run.  A lane's E
// consecutive columns lie inside one block and are written as whole 16-byte
// vectors.
__device__ __forceinline__ int64_t part_index(int64_t col, int64_t strip, int64_t G)
{
    return ((col / RN_PART_COLS) * G + strip) * RN_PART_COLS + (col % RN_PART_COLS);
}

// E consecutive fp32 values to p: 16-byte stores when p allows them (the
// workspace always does; dw itself, written directly by a single strip, need
// only be 4-byte aligned).
template <int E>
__device__ __forceinline__ void store_floats(float* p, const float* v, bool vec)
{
    if (vec) {
#pragma unroll
        for (int k = 0; k < E; k += 4) {
            u32x4 w = {__float_as_uint(v[k]), __float_as_uint(v[k + 1]), __float_as_uint(v[k + 2]),
                       __float_as_uint(v[k + 3])};
            *reinterpret_cast<u32x4*>(p + k) = w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k) p[k] = v[k];
    }
}

template <int XT, int WT, int LPRC, int NV, int WGMAX, bool NT, int PD, bool ST, bool RES>
__global__ __launch_bounds__(WGMAX) void k_rmsnorm_bwd(BwdArgs a)
{
    constexpr int E = Elems<XT>::value;
    constexpr int XB = (XT == DT_BF16) ? 2 : 4;
    constexpr int WPER = (WT == DT_F32) ? 4 : 8;    // w values per 16-byte word
    constexpr int WCH = E / WPER;                   // w words per x chunk
    constexpr int HALF = E / 2;                     // accumulators staged per LDS pass

    __shared__ float red[2][16];
    __shared__ double stage[WGMAX * HALF];

    const Rows<LPRC> R(a.lpr);
    const int lane = R.lane, lpr = R.lpr, gpw = R.gpw;
    const int tid = threadIdx.x;
    const int nch = a.nch;
    const int64_t G = gridDim.x;
    const int64_t strip = xcd_chunk(blockIdx.x, G);

    const RowWalk W = row_walk(a.interleave != 0, strip, G, a.T, gpw, R.grp);
    const int n_it = W.n_it;

    int cix[NV];
    bool cok[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + lpr * i;
        cok[i] = c < nch;
        cix[i] = cok[i] ? c : nch - 1;
    }

    // w for this lane's columns: packed words in registers, unpacked at use.
    u32x4 wr[NV][WCH];
    {
        const u32x4* wp = static_cast<const u32x4*>(a.w);
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int k = 0; k < WCH; ++k) wr[i][k] = keep_if(cok[i], wp[cix[i] * WCH + k]);
    }
    auto w_of = [&](int i, float* wf) {
#pragma unroll
        for (int k = 0; k < WCH; ++k) {
            u32x4 t = wr[i][k];
            if constexpr (NV > 1) opaque(t);     // one vector per lane: keep w unpacked
            unpack<WT>(t, wf + k * WPER);
        }
    };

    double acc[NV][E];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[i][e] = 0.0;

    const char* gbase = static_cast<const char*>(a.dy);
    const char* xbase = static_cast<const char*>(a.x);
    const char* grbase = static_cast<const char*>(a.gres);
    char* dxbase = static_cast<char*>(a.dx);

    struct RowBuf {
        u32x4 g[NV], x[NV];
        u32x4 gr[RES ? NV : 1];
        float rs;
    };

    // Rows of this group: lo + grp + it * gpw; past the end of the strip the
    // address is clamped to the strip's last row, whose values then enter with
    // rstd = 0 (no dot product, no dw contribution) and are not stored.  The
    // loaded registers are not touched until they are used, so the next row's
    // loads stay in flight while the current row is processed.
    // A row group of 64 lanes or more spans whole wavefronts, so its row is the
    // same in every lane of a wavefront: row addresses and rstd are then scalar.
    auto row_of = [&](int it) {
        const int64_t r = W.row(it);
        return LPRC == 64 ? wave_uniform(r) : r;
    };
    auto load = [&](RowBuf& b, int it) {
        const int64_t rr = W.clamp(row_of(it));
        b.rs = a.rstd[rr];
        const u32x4* grow = reinterpret_cast<const u32x4*>(gbase + rr * a.lddy * XB);
        const u32x4* xrow = reinterpret_cast<const u32x4*>(xbase + rr * a.ldx * XB);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            b.g[i] = ld16<NT>(grow + cix[i]);
            b.x[i] = ld16<NT>(xrow + cix[i]);
        }
        if constexpr (RES) {
            const u32x4* rrow = reinterpret_cast<const u32x4*>(grbase + rr * a.ldgr * XB);
#pragma unroll
            for (int i = 0; i < NV; ++i) b.gr[i] = ld16<NT>(rrow + cix[i]);
        }
    };

    auto process = [&](const RowBuf& b, int it) {
        const int64_t r = row_of(it);
        const bool valid = W.valid(r);
        const float rs = valid ? b.rs : 0.0f;
        // With one vector per lane the unpacked row (g, x, g*w) stays in
        // registers between the two passes; wider lanes unpack it again.
        constexpr bool KEEP = (NV == 1);
        float xk[KEEP ? NV : 1][E], gwk[KEEP ? NV : 1][E];
        // Rows of two vectors per lane, bf16: the products g*x (exact in
        // fp32) are taken here and added into the FP64 accumulators after the
        // row's dx is stored, pinned there (below), off the path to the row
        // reduction's barrier.  Left to itself the compiler defers the
        // accumulation of a whole unrolled block of rows past its last store,
        // which in this form costs spills; with one vector per lane that
        // deferral fits in registers and measured as fast or faster, so those
        // forms (and fp32 rows) add their products here and leave the
        // schedule to the compiler.
        constexpr bool PIN = (NV > 1);
        constexpr bool DW_LATE = PIN && (XT == DT_BF16);
        float pgx[DW_LATE ? NV : 1][E];
        // s = sum_j g*w*x (the row's dot product is rstd * s), and the exact
        // dw contributions of this row.
        const double rsd = (double)rs;
        float sgwx = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float g[E], x[E], wf[E];
            unpack<XT>(keep_if(cok[i], b.g[i]), g);    // clamped duplicate chunks add nothing
            unpack<XT>(b.x[i], x);
            w_of(i, wf);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float gw = g[e] * wf[e];
                sgwx = __builtin_fmaf(gw, x[e], sgwx);
                if constexpr (DW_LATE)
                    pgx[i][e] = g[e] * x[e];
                else if constexpr (XT == DT_BF16)
                    acc[i][e] = __builtin_fma((double)(g[e] * x[e]), rsd, acc[i][e]);
                else
                    acc[i][e] = __builtin_fma((double)g[e] * (double)x[e], rsd, acc[i][e]);
                if constexpr (KEEP) {
                    xk[i][e] = x[e];
                    gwk[i][e] = gw;
                }
            }
        }
        sgwx = R.sum(sgwx, red, it);
        // dx = rstd*(g*w - c*xhat) with c = rstd*s/H and xhat = rstd*x:
        //    = rstd*(g*w) - (c*rstd*rstd)*x
        const float cm = rs * sgwx * a.inv_h;
        const float k2 = cm * rs * rs;
        if (valid) {
            u32x4* dxrow = reinterpret_cast<u32x4*>(dxbase + r * a.lddx * XB);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float o[E];
                if constexpr (KEEP) {
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(rs, gwk[i][e], -k2 * xk[i][e]);
                } else {
                    float g[E], x[E], wf[E];
                    u32x4 gc = b.g[i], xc = b.x[i];
                    opaque(gc);
                    opaque(xc);
                    unpack<XT>(gc, g);
                    unpack<XT>(xc, x);
                    w_of(i, wf);
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(rs, g[e] * wf[e], -k2 * x[e]);
                }
                if constexpr (RES) {
                    float gr[E];
                    unpack<XT>(b.gr[i], gr);
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] += gr[e];
                }
                if (cok[i]) st16<NT>(dxrow + cix[i], pack<XT>(o));
            }
        }
        if constexpr (DW_LATE) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[i][e] = __builtin_fma((double)pgx[i][e], rsd, acc[i][e]);
        }
        if constexpr (PIN) {
            // The row's dw contributions are added now, not deferred past the
            // next rows (which would keep this row's products live meanwhile).
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int e = 0; e < E; ++e) settle(acc[i][e]);
        }
    };

    // PD row buffers in a ring: the g, x and rstd of the next PD-1 rows are in
    // flight while the current row is reduced and written.  ST selects the
    // steady form.  The plain streaming launch runs three buffers in the steady
    // form; the residual one, which loads a third row per row, runs two (one
    // row in flight), measured faster or equal on MI355X at every shape tried; few rows
    // and rows wider than 1024 chunks keep two buffers in the guarded form,
    // measured the same or 0.1-0.25 us faster per call at few rows.
    row_pipeline<PD, ST, RowBuf>(n_it, load, process);

    // Emit this strip's dw partial: the gpw row groups' accumulators are
    // combined in a fixed order (group 0, 1, ...) in FP64 and rounded once to
    // fp32.  Groups 1.. stage their values through LDS, HALF per lane per
    // pass; group 0 adds them to its own and writes whole vectors.
    const bool vec = a.part_vec != 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + lpr * i;
        float outv[E];
        if (gpw == 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) outv[e] = (float)acc[i][e];
        } else {
#pragma unroll
            for (int h0 = 0; h0 < E; h0 += HALF) {
                if (R.grp > 0) {
#pragma unroll
                    for (int e = 0; e < HALF; ++e) stage[tid * HALF + e] = acc[i][h0 + e];
                }
                __syncthreads();
                if (R.grp == 0) {
#pragma unroll
                    for (int e = 0; e < HALF; ++e) {
                        double s = 0.0 + acc[i][h0 + e];
                        for (int q = 1; q < gpw; ++q) s += stage[(q * lpr + lane) * HALF + e];
                        outv[h0 + e] = (float)s;
                    }
                }
                __syncthreads();
            }
        }
        if (R.grp == 0 && c < nch) store_floats<E>(a.part + part_index((int64_t)c * E, strip, G), outv, vec);
    }
}

// dw[j] = fp32( sum over g = 0..G-1 of the strip partials of column j ), in
// FP64 and a fixed order.  One work-group per block of 16 columns, whose G x 16
// partials are contiguous.  Thread t reads 16-byte vectors (four columns,
// quad t % 4) of the strips g = t/4, t/4 + 64, t/4 + 128, ... and adds them in
// that order, issuing four loads before the first add (the partials were just
// written by other CUs, so each round trip goes to memory); the 64 sums of a
// column are then added as four runs of 16 (strip lanes 0-15, 16-31, ...) and
// the four run totals in order.
__global__ __launch_bounds__(256) void k_dw_reduce(ReduceArgs a)
{
    __shared__ double red[64][RN_PART_COLS + 1];
    __shared__ double red2[4][RN_PART_COLS];
    const int t = threadIdx.x;
    const int cq = t & 3, sl = t >> 2;
    const int64_t blk = blockIdx.x;
    const int64_t G = a.G;
    const u32x4* p = reinterpret_cast<const u32x4*>(a.part + blk * G * RN_PART_COLS) + cq;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    auto add = [&](const u32x4& v) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += (double)__uint_as_float(v[k]);
    };
    int64_t g = sl;
    for (; g + 192 < G; g += 256) {
        const u32x4 v0 = p[g * 4], v1 = p[(g + 64) * 4], v2 = p[(g + 128) * 4], v3 = p[(g + 192) * 4];
        add(v0);
        add(v1);
        add(v2);
        add(v3);
    }
    for (; g < G; g += 64) add(p[g * 4]);
#pragma unroll
    for (int k = 0; k < 4; ++k) red[sl][cq * 4 + k] = acc[k];
    __syncthreads();
    if (t < 64) {
        const int c = t & 15, run = t >> 4;
        double u = 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) u += red[run * 16 + k][c];
        red2[run][c] = u;
    }
    __syncthreads();
    const int64_t col = blk * RN_PART_COLS + t;
    if (t < 16 && col < a.H) a.dw[col] = (float)(((red2[0][t] + red2[1][t]) + red2[2][t]) + red2[3][t]);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Variant table and dispatch.
// ---------------------------------------------------------------------------
template <int XT, int WT, int LPRC, int NV, int WGMAX, bool RES>
static hipError_t bwd_go(const BwdArgs& a, const Policy& p, hipStream_t s)
{
    const dim3 g((unsigned)p.grid), b(p.wgs);
    const int pd = (p.flags >> 4) & 7;
    // The residual form is compiled with streaming accesses only.
    const bool nt = RES || (p.flags & RN_FLAG_NT) != 0;
    if constexpr (NV <= 2) {
        // pipeline depth and form are launch choices
        if (pd == 3) {
            if (nt) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, true, 3, true, RES>), g, b, 0, s, a);
            else if constexpr (!RES) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, false, 3, true, false>), g, b, 0, s, a);
            return hipGetLastError();
        }
        if constexpr (LPRC == 64 && NV == 1) {
            if (pd == 4) {
                if (nt) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, true, 4, true, RES>), g, b, 0, s, a);
                else if constexpr (!RES) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, false, 4, true, false>), g, b, 0, s, a);
                return hipGetLastError();
            }
        }
        if constexpr (RES && WGMAX <= 512) {
            // two buffers in the steady form: the residual streaming launch
            // (groups of at most 512 lanes)
            if (pd == 2 && (p.flags & RN_FLAG_STEADY)) {
                hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, true, 2, true, true>), g, b, 0, s, a);
                return hipGetLastError();
            }
        }
    }
    if (nt) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, true, 2, false, RES>), g, b, 0, s, a);
    else if constexpr (!RES) hipLaunchKernelGGL((k_rmsnorm_bwd<XT, WT, LPRC, NV, WGMAX, false, 2, false, false>), g, b, 0, s, a);
    return hipGetLastError();
}

// (group class, vectors per lane, largest work-group) triples compiled.
// The first match serves a launch, so the 512-thread bounds (a 256-register
// budget per lane) come before the 1024-thread ones (128 registers).
#define RN_BWD_VARIANTS(X) X(16, 1, 512) X(16, 1, 1024) X(32, 1, 512) X(32, 1, 1024) X(64, 1, 512) X(64, 1, 1024) \
    X(64, 2, 512) X(64, 2, 1024)

bool bwd_variant_exists(int lprc, int nv, int wgs)
{
#define X(C, N, W) if (lprc == C && nv == N && wgs <= W) return true;
    RN_BWD_VARIANTS(X)
#undef X
    return false;
}

template <int XT, int WT, bool RES>
static hipError_t bwd_dispatch(const BwdArgs& a, const Policy& p, hipStream_t s)
{
    const int lprc = p.lpr < 64 ? p.lpr : 64;
#define X(C, N, W) if (lprc == C && p.nv == N && p.wgs <= W) return bwd_go<XT, WT, C, N, W, RES>(a, p, s);
    RN_BWD_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

template <bool RES>
static hipError_t bwd_dtypes(const BwdArgs& a, int x_dtype, int w_dtype, const Policy& p, hipStream_t s)
{
    if (x_dtype == DT_BF16 && w_dtype == DT_BF16) return bwd_dispatch<DT_BF16, DT_BF16, RES>(a, p, s);
    if (x_dtype == DT_BF16 && w_dtype == DT_F32) return bwd_dispatch<DT_BF16, DT_F32, RES>(a, p, s);
    if (x_dtype == DT_F32 && w_dtype == DT_F32) return bwd_dispatch<DT_F32, DT_F32, RES>(a, p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int x_dtype, int w_dtype, int residual, const Policy& p, hipStream_t s)
{
    return residual ? bwd_dtypes<true>(a, x_dtype, w_dtype, p, s) : bwd_dtypes<false>(a, x_dtype, w_dtype, p, s);
}

hipError_t launch_bwd_reduce(const ReduceArgs& a, hipStream_t s)
{
    const unsigned grid = (unsigned)((a.H + RN_PART_COLS - 1) / RN_PART_COLS);
    hipLaunchKernelGGL(k_dw_reduce, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

} // namespace rn

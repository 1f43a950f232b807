// rn_fp8.hip -- fused residual add + RMSNorm + FP8 e4m3 1x128 block quant (gfx950).
//
// Operation ([F] = FlashInfer PR #4480 "Add FusedAddRMSNormFP8BlockQuant",
// description: Kernel and API; review thread: scale layout and e4m3 only):
//   h = bf16(x + residual)  -> written back into residual (pre-norm sum)
//   rstd = 1/sqrt(mean(h^2) + eps)
//   n = bf16(h * rstd * w)  -> normed_out
//   per 1x128 block: s = amax|n| / 448 (fp32) -> block_scale[k * ld + row]
//   out = e4m3fn(n / s), quantised from the bf16-rounded n, so out is exactly
//   a re-quantisation of normed_out.
//
// Mapping.  One row per group of LPR lanes, rows of a work-group's chunk
// taken GPW at a time; the next row's x and residual are loaded as soon as
// the current row's h is formed, overlapping its normalize/quantize/store.  Chunk c (8 bf16) belongs to lane c % LPR, so for
// LPR in {16, 32, 64, ...} a 1x128 block (16 chunks) is exactly one 16-lane
// DPP row: the block amax is four DPP max steps on packed-magnitude integers,
// with no LDS.  The row (h, then n) stays in registers; HBM sees x and
// residual read once, residual, normed and the codes written once.
//
// Quotient n/s.  The codes must equal e4m3(fl(n/s)) with fl the IEEE fp32
// quotient.  Per block the reciprocal r of s is formed once (hardware rcp and
// one Newton step); per element y = n*r is corrected with the exact FMA
// residual e = n - s*y to q = y + e*r, which is the correctly rounded quotient
// for every (n, s) pair that can occur (|n| <= amax, s = fl(amax/448) with
// amax a bf16 value): the library's self-test checks all such pairs against
// the IEEE division exhaustively.  Blocks whose scale is below 2^-100 (where
// 1/s would overflow) take the IEEE division instead.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// Correctly rounded n / s for s >= 2^-100 and |n| <= 448 * s (see above).
__device__ __forceinline__ float quot_fast(float n, float s, float r)
{
    const float y = n * r;
    const float e = __builtin_fmaf(-s, y, n);
    const float q = __builtin_fmaf(e, r, y);
    return __builtin_copysignf(q, n);
}

__device__ __forceinline__ float recip_refined(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// Four e4m3 codes (round to nearest even) packed little-endian into a word.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Codes of one 8-value chunk of bf16 normed values n (packed in nv) given the
// block scale s.  Exported to the self-test kernel below.
__device__ __forceinline__ u32x2 quant_chunk(const u32x4& nv, float s)
{
    float q[8];
    if (s >= 0x1p-100f) {
        const float r = recip_refined(s);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[2 * k] = quot_fast(bf16lo(nv[k]), s, r);
            q[2 * k + 1] = quot_fast(bf16hi(nv[k]), s, r);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[2 * k] = bf16lo(nv[k]) / s;
            q[2 * k + 1] = bf16hi(nv[k]) / s;
        }
    }
    u32x2 o;
    o[0] = cvt4_e4m3(q[0], q[1], q[2], q[3]);
    o[1] = cvt4_e4m3(q[4], q[5], q[6], q[7]);
    if (s == 0.0f) o = u32x2{0u, 0u};    // all-zero block: scale 0, codes 0x00
    return o;
}

// Largest |value| bit pattern among the 8 bf16 of a chunk (bf16 magnitudes
// order like their bit patterns).
__device__ __forceinline__ uint32_t chunk_absmax_bits(const u32x4& v)
{
    u16x2 m = __builtin_bit_cast(u16x2, v[0] & 0x7fff7fffu);
#pragma unroll
    for (int k = 1; k < 4; ++k) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[k] & 0x7fff7fffu));
    return (uint32_t)max(m[0], m[1]);
}

template <int LPRC, int NV, int WGMAX, bool NT>
__global__ __launch_bounds__(WGMAX) void k_add_rmsnorm_fp8(Fp8Args a)
{
    static_assert(LPRC % 16 == 0, "a 1x128 block must be one 16-lane DPP row");

    __shared__ float red[2][16];

    const Rows<LPRC> R(a.lpr);
    const int lane = R.lane, lpr = R.lpr, gpw = R.gpw;
    const int nch = a.nch;

    const RowWalk W = row_walk(a.interleave != 0, xcd_chunk(blockIdx.x, gridDim.x), gridDim.x, a.T, gpw, R.grp);
    const int n_it = W.n_it;

    int cix[NV];
    bool cok[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + lpr * i;
        cok[i] = c < nch;
        cix[i] = cok[i] ? c : nch - 1;
    }

    u32x4 wv[NV];
    {
        const u32x4* wp = static_cast<const u32x4*>(a.w);
#pragma unroll
        for (int i = 0; i < NV; ++i) wv[i] = keep_if(cok[i], wp[cix[i]]);
    }

    const char* xbase = static_cast<const char*>(a.x);
    char* rbase = static_cast<char*>(a.res);
    char* nbase = static_cast<char*>(a.normed);

    // Loads of a row's x and residual; past the chunk end the address is
    // clamped to the chunk's last row (nothing is stored for it).  The loaded
    // registers are left untouched until they are used.
    u32x4 xv[NV], rv[NV];
    auto load = [&](int it) {
        const int64_t rr = W.clamp(W.row(it));
        const u32x4* xrow = reinterpret_cast<const u32x4*>(xbase + rr * a.ldx * 2);
        const u32x4* rrow = reinterpret_cast<const u32x4*>(rbase + rr * a.ldr * 2);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            xv[i] = ld16<NT>(xrow + cix[i]);
            rv[i] = ld16<NT>(rrow + cix[i]);
        }
    };

    load(0);
    for (int it = 0; it < n_it; ++it) {
        const int64_t r = W.row(it);
        const bool valid = W.valid(r);

        // h = bf16(x + r): the fp32 sum of two bf16 values rounds to the
        // same bf16 as their exact sum.
        u32x4 hv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                hv[i][k] = pack_bf16x2(bf16lo(xv[i][k]) + bf16lo(rv[i][k]), bf16hi(xv[i][k]) + bf16hi(rv[i][k]));
            hv[i] = keep_if(cok[i], hv[i]);     // clamped duplicate chunks are zero
        }

        // x and residual of this row are consumed: the next row's loads go
        // into the same registers and overlap the rest of this row.
        if (it + 1 < n_it) load(it + 1);

        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float l = bf16lo(hv[i][k]), h = bf16hi(hv[i][k]);
                ss = __builtin_fmaf(l, l, ss);
                ss = __builtin_fmaf(h, h, ss);
            }
        }
        if (valid) {
            u32x4* rrow = reinterpret_cast<u32x4*>(rbase + r * a.ldr * 2);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (cok[i]) st16<NT>(rrow + cix[i], hv[i]);
        }
        ss = R.sum(ss, red, it);
        const float rs = 1.0f / __builtin_sqrtf(ss / (float)a.H + a.eps);

        u32x4* nrow = reinterpret_cast<u32x4*>(nbase + r * a.ldn * 2);
        u32x2* orow = reinterpret_cast<u32x2*>(a.out + r * a.ldo);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            u32x4 nv;
            u32x4 wc = wv[i];
            opaque(wc);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                nv[k] = pack_bf16x2((bf16lo(hv[i][k]) * rs) * bf16lo(wc[k]), (bf16hi(hv[i][k]) * rs) * bf16hi(wc[k]));
            const uint32_t mb = max16_u32(chunk_absmax_bits(nv));
            const float amax = __uint_as_float(mb << 16);
            const float s = amax / 448.0f;
            const u32x2 q = quant_chunk(nv, s);
            if (valid && cok[i]) {
                st16<NT>(nrow + cix[i], nv);
                st8<NT>(orow + cix[i], q);
                if ((lane & 15) == 0) a.scale[(int64_t)(cix[i] >> 4) * a.scale_ld + r] = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Variant table and dispatch.
// ---------------------------------------------------------------------------
template <int LPRC, int NV, int WGMAX>
static hipError_t fp8_go(const Fp8Args& a, const Policy& p, hipStream_t s)
{
    if (p.flags & RN_FLAG_NT)
        hipLaunchKernelGGL((k_add_rmsnorm_fp8<LPRC, NV, WGMAX, true>), dim3((unsigned)p.grid), dim3(p.wgs), 0, s, a);
    else
        hipLaunchKernelGGL((k_add_rmsnorm_fp8<LPRC, NV, WGMAX, false>), dim3((unsigned)p.grid), dim3(p.wgs), 0, s, a);
    return hipGetLastError();
}

#define RN_FP8_VARIANTS(X) X(16, 1, 256) X(32, 1, 256) X(64, 1, 256) X(64, 2, 256) X(64, 3, 256)        \
    X(64, 4, 256) X(64, 5, 256) X(64, 6, 256) X(64, 7, 256) X(64, 8, 256) X(64, 5, 512) X(64, 6, 512)  \
    X(64, 7, 512) X(64, 8, 512)

bool fp8_variant_exists(int lprc, int nv, int wgs)
{
#define X(C, N, W) if (lprc == C && nv == N && wgs <= W) return true;
    RN_FP8_VARIANTS(X)
#undef X
    return false;
}

hipError_t launch_fp8(const Fp8Args& a, const Policy& p, hipStream_t s)
{
    const int lprc = p.lpr < 64 ? p.lpr : 64;
#define X(C, N, W) if (lprc == C && p.nv == N && p.wgs <= W) return fp8_go<C, N, W>(a, p, s);
    RN_FP8_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Self-test of the quantisation step: for every positive finite bf16 amax and
// every bf16 n with |n| <= amax, compare the kernel's codes (quant_chunk) with
// e4m3(n / s) computed with the IEEE fp32 division.  Counts mismatches.
// Grid: one work-group per amax pattern (blockIdx.x + a_lo); each thread walks
// the n patterns with stride 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_selftest(uint32_t a_lo, unsigned long long* mismatches,
                                                        uint32_t* first_bad)
{
    const uint32_t abits = a_lo + blockIdx.x;              // 0x0001 .. 0x7f7f
    const float amax = __uint_as_float(abits << 16);
    const float s = amax / 448.0f;
    unsigned long long bad = 0;
    for (int p = 0; p < 2; ++p) {
        for (uint32_t m = threadIdx.x * 8; m <= abits; m += 256 * 8) {
            // 8 consecutive magnitudes m .. m+7 (clamped to abits); the sign
            // alternates, and the second pass flips it
            u32x4 nv;
            uint32_t b[8];
            float qi[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t mag = m + k;
                if (mag > abits) mag = abits;
                b[k] = mag | (((k + p) & 1) ? 0x8000u : 0u);
                qi[k] = __uint_as_float(b[k] << 16) / s;   // IEEE fp32 division
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) nv[k] = b[2 * k] | (b[2 * k + 1] << 16);
            const u32x2 q = quant_chunk(nv, s);
            const uint32_t r0 = cvt4_e4m3(qi[0], qi[1], qi[2], qi[3]);
            const uint32_t r1 = cvt4_e4m3(qi[4], qi[5], qi[6], qi[7]);
            if (q[0] != r0 || q[1] != r1) {
                ++bad;
                atomicMin(first_bad, (abits << 16) | m);
            }
        }
    }
    if (bad) atomicAdd(mismatches, bad);
}

// Codes of n fp32 values through the same conversion the producer uses.
__global__ __launch_bounds__(256) void k_cvt_e4m3(const float* in, uint8_t* out, int64_t n)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 3 < n) {
        const uint32_t w = cvt4_e4m3(in[i], in[i + 1], in[i + 2], in[i + 3]);
        out[i] = (uint8_t)w; out[i + 1] = (uint8_t)(w >> 8);
        out[i + 2] = (uint8_t)(w >> 16); out[i + 3] = (uint8_t)(w >> 24);
    } else {
        for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)cvt4_e4m3(in[j], 0.0f, 0.0f, 0.0f);
    }
}

} // namespace rn

// Host hook for the self-test (declared in the public header).
extern "C" int rn_selftest_quant(uint32_t a_lo, uint32_t a_hi, unsigned long long* d_mismatches,
                                 uint32_t* d_first_bad, void* stream)
{
    if (a_lo < 1 || a_hi > 0x7f7f || a_lo > a_hi || !d_mismatches || !d_first_bad) return 2;
    hipLaunchKernelGGL(rn::k_quant_selftest, dim3(a_hi - a_lo + 1), dim3(256), 0, (hipStream_t)stream,
                       a_lo, d_mismatches, d_first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

extern "C" int rn_selftest_cvt_e4m3(const float* d_in, uint8_t* d_out, int64_t n, void* stream)
{
    if (n < 0 || (n > 0 && (!d_in || !d_out))) return 1;
    if (n == 0) return 0;
    const int64_t nthreads = (n + 3) / 4;
    hipLaunchKernelGGL(rn::k_cvt_e4m3, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, d_in, d_out, n);
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

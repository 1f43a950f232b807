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
// Quotient n/s.  The codes must equal fp8(fl(n/s)) with fl the IEEE fp32
// quotient.  Per block the reciprocal r of s is formed once (hardware rcp and
// one Newton step); per element y = n*r is corrected with the exact FMA
// residual e = n - s*y to q = y + e*r, which is the correctly rounded quotient
// for every (n, s) pair that can occur (|n| <= amax, s = fl(amax/MAX) with
// amax a bf16 or fp16 value): the library's self-test checks all such pairs
// against the IEEE division exhaustively.  Blocks whose scale is below
// 2^-100 (where 1/s would overflow) take the IEEE division instead.
//
// Variants ([F] description: the block-scaled sibling of the per-tensor
// FusedAddRMSNormQuant; its tests over fp16 and bf16 inputs; review thread:
// the bound 448 tied to the output type):
//   XT   bf16 or fp16 rows (h and n rounded to that type)
//   FMT  e4m3 (MAX 448) or e5m2 (MAX 57344) codes
//   TSC  a given per-tensor scale s for every element instead of block
//        scales.  With r = fl(1/s) (IEEE, once per kernel) the same
//        correction gives the correctly rounded quotient whenever the
//        quotient is a normal fp32 number and the residual does not fall
//        below the fp32 range (Markstein's theorem: r is the correctly
//        rounded reciprocal and y is within one ulp of n/s); nonzero |n| below
//        2^-100 take the IEEE division instead.  Quotients then saturate at
//        +-MAX before the conversion.
#include "../../include/rmsnorm_gfx950.h"
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

constexpr int FMT_E4M3 = 0;
constexpr int FMT_E5M2 = 1;

template <int FMT> struct Fp8Max { static constexpr float value = FMT == FMT_E5M2 ? 57344.0f : 448.0f; };

// n / s from y = n*r and the exact FMA residual (see above).
__device__ __forceinline__ float quot_fix(float n, float s, float r, float y)
{
    const float e = __builtin_fmaf(-s, y, n);
    const float q = __builtin_fmaf(e, r, y);
    return __builtin_copysignf(q, n);
}

// Correctly rounded n / s for s >= 2^-100 and |n| <= 448 * s (see above).
__device__ __forceinline__ float quot_fast(float n, float s, float r) { return quot_fix(n, s, r, n * r); }

__device__ __forceinline__ float recip_refined(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// Four fp8 codes (round to nearest even) packed little-endian into a word.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d)
{
    int w;
    if constexpr (FMT == FMT_E5M2) {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    }
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) { return cvt4<FMT_E4M3>(a, b, c, d); }

// The quotient of one element, as the codes use it.  fast: s >= 2^-100 (the
// reciprocal r is finite).  Per-tensor form: quotients saturate at +-MAX, and
// a nonzero |n| below 2^-100 takes the IEEE division (the FMA residual of the
// correction could fall below the fp32 range there; see tiny_n).
template <int FMT, bool TSC>
__device__ __forceinline__ float quot_elem(float n, float s, float r, bool fast)
{
    constexpr float MX = Fp8Max<FMT>::value;
    float q;
    if (fast) {
        const float y = n * r;
        q = quot_fix(n, s, r, y);
        if constexpr (TSC)   // |y| >= 2*MAX is far beyond saturation (and y may have overflowed)
            q = __builtin_fabsf(y) < 2.0f * MX ? __builtin_fminf(__builtin_fmaxf(q, -MX), MX)
                                               : __builtin_copysignf(MX, n);
    } else {
        q = n / s;
        if constexpr (TSC) q = __builtin_fminf(__builtin_fmaxf(q, -MX), MX);
    }
    return q;
}

// Per-tensor form: |n| nonzero and below 2^-100 (rare; handled off the fast path).
__device__ __forceinline__ bool tiny_n(float n)
{
    const float an = __builtin_fabsf(n);
    return an < 0x1p-100f && an != 0.0f;
}

// Codes of one 8-value chunk of 16-bit normed values (packed in nv) given
// the scale s and, for a per-tensor scale, r = fl(1/s).  A scale that is not
// a positive number (an all-zero block) gives codes 0x00.
template <int XT, int FMT, bool TSC>
__device__ __forceinline__ u32x2 quant_chunk(const u32x4& nv, float s, float r_tensor)
{
    const bool fast = s >= 0x1p-100f;
    const float r = TSC ? r_tensor : (fast ? recip_refined(s) : 0.0f);
    float q[8];
    bool tiny = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float n = (k & 1) ? hi16<XT>(nv[k >> 1]) : lo16<XT>(nv[k >> 1]);
        q[k] = quot_elem<FMT, TSC>(n, s, r, fast);
        if constexpr (TSC) tiny |= tiny_n(n);
    }
    if constexpr (TSC) {
        if (tiny && fast) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float n = (k & 1) ? hi16<XT>(nv[k >> 1]) : lo16<XT>(nv[k >> 1]);
                if (tiny_n(n)) q[k] = quot_elem<FMT, TSC>(n, s, r, false);
            }
        }
    }
    u32x2 o;
    o[0] = cvt4<FMT>(q[0], q[1], q[2], q[3]);
    o[1] = cvt4<FMT>(q[4], q[5], q[6], q[7]);
    if (!(s > 0.0f)) o = u32x2{0u, 0u};
    return o;
}

// Largest |value| bit pattern among the 8 16-bit values of a chunk (bf16 and
// fp16 magnitudes order like their bit patterns).
__device__ __forceinline__ uint32_t chunk_absmax_bits(const u32x4& v)
{
    u16x2 m = __builtin_bit_cast(u16x2, v[0] & 0x7fff7fffu);
#pragma unroll
    for (int k = 1; k < 4; ++k) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[k] & 0x7fff7fffu));
    return (uint32_t)max(m[0], m[1]);
}

template <int XT, int FMT, bool TSC, int LPRC, int NV, int WGMAX, bool NT>
__global__ __launch_bounds__(WGMAX) void k_add_rmsnorm_fp8(Fp8Args a)
{
    static_assert(LPRC % 16 == 0, "a 1x128 block must be one 16-lane DPP row");
    constexpr float MX = Fp8Max<FMT>::value;

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

    // A per-tensor scale and its correctly rounded reciprocal, once.
    float ts = 0.0f, tr = 0.0f;
    if constexpr (TSC) {
        ts = a.tscale[0];
        tr = 1.0f / ts;
    }

    const char* xbase = static_cast<const char*>(a.x);
    char* rbase = static_cast<char*>(a.res);
    char* nbase = static_cast<char*>(a.normed);
    const bool want_normed = nbase != nullptr;

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

        // h = round(x + r): the fp32 sum of two bf16 (or fp16) values rounds
        // to the same 16-bit value as their exact sum.
        u32x4 hv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                hv[i][k] = pack16x2<XT>(lo16<XT>(xv[i][k]) + lo16<XT>(rv[i][k]), hi16<XT>(xv[i][k]) + hi16<XT>(rv[i][k]));
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
                const float l = lo16<XT>(hv[i][k]), h = hi16<XT>(hv[i][k]);
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
                nv[k] = pack16x2<XT>((lo16<XT>(hv[i][k]) * rs) * lo16<XT>(wc[k]),
                                     (hi16<XT>(hv[i][k]) * rs) * hi16<XT>(wc[k]));
            float s = ts;
            if constexpr (!TSC) {
                const uint32_t mb = max16_u32(chunk_absmax_bits(nv));
                const float amax = XT == DT_F16 ? f16lo(mb) : bf16lo(mb);
                s = amax / MX;
            }
            const u32x2 q = quant_chunk<XT, FMT, TSC>(nv, s, tr);
            if (valid && cok[i]) {
                if (want_normed) st16<NT>(nrow + cix[i], nv);
                st8<NT>(orow + cix[i], q);
                if constexpr (!TSC)
                    if ((lane & 15) == 0) a.scale[(int64_t)(cix[i] >> 4) * a.scale_ld + r] = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Variant table and dispatch.  The bf16 / e4m3 / block-scale producer has
// both access forms; the other variants are compiled with streaming
// accesses only.
// ---------------------------------------------------------------------------
template <int XT, int FMT, bool TSC, int LPRC, int NV, int WGMAX>
static hipError_t fp8_go(const Fp8Args& a, const Policy& p, hipStream_t s)
{
    constexpr bool BASE = XT == DT_BF16 && FMT == FMT_E4M3 && !TSC;
    const dim3 g((unsigned)p.grid), b(p.wgs);
    if (!BASE || (p.flags & RN_FLAG_NT))
        hipLaunchKernelGGL((k_add_rmsnorm_fp8<XT, FMT, TSC, LPRC, NV, WGMAX, true>), g, b, 0, s, a);
    else if constexpr (BASE)
        hipLaunchKernelGGL((k_add_rmsnorm_fp8<XT, FMT, TSC, LPRC, NV, WGMAX, false>), g, b, 0, s, a);
    return hipGetLastError();
}

#define RN_FP8_VARIANTS(X) X(16, 1, 256) X(32, 1, 256) X(64, 1, 256) X(64, 2, 256) X(64, 3, 256)        \
    X(64, 4, 256) X(64, 5, 256) X(64, 6, 256) X(64, 7, 256) X(64, 8, 256) X(64, 2, 512) X(64, 3, 512)  \
    X(64, 4, 512) X(64, 5, 512) X(64, 6, 512) X(64, 7, 512) X(64, 8, 512)

bool fp8_variant_exists(int lprc, int nv, int wgs)
{
#define X(C, N, W) if (lprc == C && nv == N && wgs <= W) return true;
    RN_FP8_VARIANTS(X)
#undef X
    return false;
}

template <int XT, int FMT, bool TSC>
static hipError_t fp8_dispatch(const Fp8Args& a, const Policy& p, hipStream_t s)
{
    const int lprc = p.lpr < 64 ? p.lpr : 64;
#define X(C, N, W) if (lprc == C && p.nv == N && p.wgs <= W) return fp8_go<XT, FMT, TSC, C, N, W>(a, p, s);
    RN_FP8_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_fp8(const Fp8Args& a, int dtype, int fmt, bool tensor_scale, const Policy& p, hipStream_t s)
{
    const int v = (dtype == DT_F16 ? 4 : 0) + (fmt == FMT_E5M2 ? 2 : 0) + (tensor_scale ? 1 : 0);
    if (dtype != DT_BF16 && dtype != DT_F16) return hipErrorInvalidValue;
    switch (v) {
    case 0: return fp8_dispatch<DT_BF16, FMT_E4M3, false>(a, p, s);
    case 1: return fp8_dispatch<DT_BF16, FMT_E4M3, true>(a, p, s);
    case 2: return fp8_dispatch<DT_BF16, FMT_E5M2, false>(a, p, s);
    case 3: return fp8_dispatch<DT_BF16, FMT_E5M2, true>(a, p, s);
    case 4: return fp8_dispatch<DT_F16, FMT_E4M3, false>(a, p, s);
    case 5: return fp8_dispatch<DT_F16, FMT_E4M3, true>(a, p, s);
    case 6: return fp8_dispatch<DT_F16, FMT_E5M2, false>(a, p, s);
    default: return fp8_dispatch<DT_F16, FMT_E5M2, true>(a, p, s);
    }
}

// ---------------------------------------------------------------------------
// Self-tests of the quantisation step.
// k_quant_selftest: for every positive finite bf16 amax and every bf16 n with
// |n| <= amax, compare the kernel's e4m3 codes (quant_chunk) with e4m3(n / s)
// computed with the IEEE fp32 division.  Counts mismatches.  Grid: one
// work-group per amax pattern (blockIdx.x + a_lo); each thread walks the n
// patterns with stride 256.
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
            const u32x2 q = quant_chunk<DT_BF16, FMT_E4M3, false>(nv, s, 0.0f);
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

// k_quotient_selftest: the producer's quotient against the IEEE division.
// Block-scale form (TSC false): for amax = the 16-bit pattern blockIdx.x +
// a_lo of dtype DT and s = fl(amax / MAX), every n of that dtype with |n| <=
// amax (both signs).  Per-tensor form: s = svals[blockIdx.x], r = fl(1/s),
// every finite n of the dtype.  For every pair the fp8 codes of the two
// quotients (the IEEE one saturated as the producer saturates) must agree;
// where |n| >= 2^-100 and the IEEE quotient is a normal number below 2 * MAX,
// the quotients must also agree bit for bit.
template <int DT, int FMT, bool TSC>
__global__ __launch_bounds__(256) void k_quotient_selftest(uint32_t a_lo, const float* svals,
                                                           unsigned long long* mismatches, uint32_t* first_bad)
{
    constexpr float MX = Fp8Max<FMT>::value;
    float s, r;
    uint32_t lim;
    if constexpr (TSC) {
        s = svals[blockIdx.x];
        r = 1.0f / s;
        lim = DT == DT_F16 ? 0x7bffu : 0x7f7fu;
    } else {
        lim = a_lo + blockIdx.x;
        const float amax = DT == DT_F16 ? f16lo(lim) : bf16lo(lim);
        s = amax / MX;
        r = s >= 0x1p-100f ? recip_refined(s) : 0.0f;
    }
    const bool fast = s >= 0x1p-100f;
    unsigned long long bad = 0;
    for (uint32_t m = threadIdx.x; m <= lim; m += 256) {
        for (int sg = 0; sg < 2; ++sg) {
            const uint32_t b = m | (sg ? 0x8000u : 0u);
            const float n = DT == DT_F16 ? f16lo(b) : bf16lo(b);
            const float exact = n / s;                       // IEEE fp32 division
            const float ref = TSC ? __builtin_fminf(__builtin_fmaxf(exact, -MX), MX) : exact;
            const float got = quot_elem<FMT, TSC>(n, s, r, fast && !(TSC && tiny_n(n)));
            const float ae = __builtin_fabsf(exact);
            bool ok = cvt4<FMT>(got, 0.0f, 0.0f, 0.0f) == cvt4<FMT>(ref, 0.0f, 0.0f, 0.0f);
            if (__builtin_fabsf(n) >= 0x1p-100f && ae >= 0x1p-126f && ae < 2.0f * MX)
                ok = ok && __float_as_uint(got) == __float_as_uint(ref);
            if (!ok) {
                ++bad;
                atomicMin(first_bad, (blockIdx.x << 16) | m);
            }
        }
    }
    if (bad) atomicAdd(mismatches, bad);
}

// Codes of n fp32 values through the conversion the producer uses.
template <int FMT>
__global__ __launch_bounds__(256) void k_cvt(const float* in, uint8_t* out, int64_t n)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 3 < n) {
        const uint32_t w = cvt4<FMT>(in[i], in[i + 1], in[i + 2], in[i + 3]);
        out[i] = (uint8_t)w; out[i + 1] = (uint8_t)(w >> 8);
        out[i + 2] = (uint8_t)(w >> 16); out[i + 3] = (uint8_t)(w >> 24);
    } else {
        for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)cvt4<FMT>(in[j], 0.0f, 0.0f, 0.0f);
    }
}

} // namespace rn

// Host hooks for the self-tests (declared in the public header).
extern "C" int rn_selftest_quant(uint32_t a_lo, uint32_t a_hi, unsigned long long* d_mismatches,
                                 uint32_t* d_first_bad, void* stream)
{
    if (a_lo < 1 || a_hi > 0x7f7f || a_lo > a_hi || !d_mismatches || !d_first_bad) return 2;
    hipLaunchKernelGGL(rn::k_quant_selftest, dim3(a_hi - a_lo + 1), dim3(256), 0, (hipStream_t)stream,
                       a_lo, d_mismatches, d_first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

extern "C" int rn_selftest_quotient(int dtype, int out_format, uint32_t a_lo, uint32_t a_hi, const float* d_scales,
                                    int64_t n_scales, unsigned long long* d_mismatches, uint32_t* d_first_bad,
                                    void* stream)
{
    if ((dtype != RN_BF16 && dtype != RN_F16) || (out_format != RN_E4M3 && out_format != RN_E5M2)) return 3;
    if (!d_mismatches || !d_first_bad) return 1;
    const uint32_t top = dtype == RN_F16 ? 0x7bffu : 0x7f7fu;
    unsigned grid;
    int tensor;
    if (d_scales) {
        if (n_scales < 1 || n_scales > 65535) return 2;
        grid = (unsigned)n_scales;
        tensor = 1;
    } else {
        if (a_lo < 1 || a_hi > top || a_lo > a_hi) return 2;
        grid = a_hi - a_lo + 1;
        tensor = 0;
    }
    const hipStream_t st = (hipStream_t)stream;
    using namespace rn;
#define RN_QST(D, F, TS) hipLaunchKernelGGL((k_quotient_selftest<D, F, TS>), dim3(grid), dim3(256), 0, st, a_lo, \
                                            d_scales, d_mismatches, d_first_bad)
    const int v = (dtype == RN_F16 ? 4 : 0) + (out_format == RN_E5M2 ? 2 : 0) + tensor;
    switch (v) {
    case 0: RN_QST(DT_BF16, FMT_E4M3, false); break;
    case 1: RN_QST(DT_BF16, FMT_E4M3, true); break;
    case 2: RN_QST(DT_BF16, FMT_E5M2, false); break;
    case 3: RN_QST(DT_BF16, FMT_E5M2, true); break;
    case 4: RN_QST(DT_F16, FMT_E4M3, false); break;
    case 5: RN_QST(DT_F16, FMT_E4M3, true); break;
    case 6: RN_QST(DT_F16, FMT_E5M2, false); break;
    default: RN_QST(DT_F16, FMT_E5M2, true); break;
    }
#undef RN_QST
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

static int launch_cvt(int fmt, const float* d_in, uint8_t* d_out, int64_t n, void* stream)
{
    if (n < 0 || (n > 0 && (!d_in || !d_out))) return 1;
    if (n == 0) return 0;
    const int64_t nthreads = (n + 3) / 4;
    const dim3 g((unsigned)((nthreads + 255) / 256));
    if (fmt == RN_E5M2)
        hipLaunchKernelGGL(rn::k_cvt<rn::FMT_E5M2>, g, dim3(256), 0, (hipStream_t)stream, d_in, d_out, n);
    else
        hipLaunchKernelGGL(rn::k_cvt<rn::FMT_E4M3>, g, dim3(256), 0, (hipStream_t)stream, d_in, d_out, n);
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

extern "C" int rn_selftest_cvt_e4m3(const float* d_in, uint8_t* d_out, int64_t n, void* stream)
{
    return launch_cvt(RN_E4M3, d_in, d_out, n, stream);
}

extern "C" int rn_selftest_cvt_e5m2(const float* d_in, uint8_t* d_out, int64_t n, void* stream)
{
    return launch_cvt(RN_E5M2, d_in, d_out, n, stream);
}

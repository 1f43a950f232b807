// rn_internal.h -- contract between the C-ABI host layer and the kernel
// translation units: launch-policy record, kernel argument blocks and the
// launcher entry points (C++ linkage, not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rn {

// A launch policy, chosen on the host from (T, H, dtypes, CU count).
struct Policy {
    int lpr;        // lanes per row group: 16, 32, 64, 128, ..., 1024
    int nv;         // 16-byte vectors per lane per row (compile-time variant)
    int wgs;        // threads per work-group
    int64_t grid;   // work-groups = row chunks
    int gpw;        // row groups per work-group (rows processed per WG pass)
    int kernel;     // variant id (for logging and tests)
    int flags;      // RN_FLAG_* bits
};

constexpr int RN_FLAG_NT = 1;    // non-temporal (streaming) loads and stores
constexpr int RN_FLAG_ILV = 2;   // interleaved row order (see RowWalk)
constexpr int RN_FLAG_STEADY = 8;   // with two row buffers: the steady prefetch form (see row_pipeline)
// bits 4-6: row-buffer pipeline depth (0 = the kernel's default)

// Forward forms (kernel template argument and launch_fwd's `mode`).
constexpr int FWD_PLAIN = 0;
constexpr int FWD_RESIDUAL = 1;   // training forward with a residual stream
constexpr int FWD_HEADS = 2;      // per-head rows (QK-norm)

struct FwdArgs {
    int lpr;                     // lanes per row group (runtime for class 64)
    int interleave;              // RN_FLAG_ILV set in the policy
    int heads;                   // per-head form: heads per token (rows = T * heads)
    uint32_t hmul; int hshift;   // per-head form: floor(r / heads) = (r * hmul) >> hshift for r < 2^31
    const void* x; int64_t ldx;
    int64_t ldxh;                // per-head form: element stride between heads of x
    int64_t ldyh;                // per-head form: element stride between heads of y
    const void* u; int64_t ldu;  // residual form: the residual input
    void* h; int64_t ldh;        // residual form: h_new = x + u, rounded to x's dtype
    const void* w;
    void* y; int64_t ldy;
    float* rstd;                 // per-head form: may be null (not stored)
    int64_t T; int H; int nch;   // T = rows; nch = H / elements-per-chunk
    float eps;
};

struct BwdArgs {
    int lpr;
    int interleave;              // RN_FLAG_ILV set in the policy
    const void* dy; int64_t lddy;
    const void* x; int64_t ldx;
    const void* w;
    const float* rstd;
    const void* gres; int64_t ldgr;   // residual form: gradient along the residual stream
    void* dx; int64_t lddx;
    float* part;                 // one fp32 dw partial per (row strip, column), column-blocked
    int part_vec;                // part is 16-byte aligned (vector stores)
    int64_t T; int H; int nch;
    float inv_h;                 // 1/H rounded to fp32
};

// dw partials are stored in blocks of this many columns (see rn_bwd.hip).
constexpr int RN_PART_COLS = 16;

struct ReduceArgs {
    const float* part;           // [ceil(H/16)][G][16]
    float* dw;                   // [H]
    int64_t G; int H;
};

struct Fp8Args {
    int lpr;
    int interleave;              // RN_FLAG_ILV set in the policy
    const void* x; int64_t ldx;
    void* res; int64_t ldr;
    const void* w;
    uint8_t* out; int64_t ldo;
    float* scale; int64_t scale_ld;   // block scales (block-scale form)
    const float* tscale;              // the given scale (per-tensor form)
    void* normed; int64_t ldn;        // may be null in the general entry point
    int64_t T; int H; int nch;
    float eps;
};

// Launchers return hipSuccess or the launch error.  They assume validated args.
// mode: FWD_PLAIN, FWD_RESIDUAL (also reads u, writes h_new) or FWD_HEADS.
// residual != 0 selects the backward that also reads g_residual.
hipError_t launch_fwd(const FwdArgs& a, int x_dtype, int w_dtype, int mode, const Policy& p, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int x_dtype, int w_dtype, int residual, const Policy& p, hipStream_t s);
hipError_t launch_bwd_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// dtype DT_BF16 / DT_F16, fmt 0 = e4m3 / 1 = e5m2, tensor_scale: the given
// per-tensor scale instead of block scales.
hipError_t launch_fp8(const Fp8Args& a, int dtype, int fmt, bool tensor_scale, const Policy& p, hipStream_t s);

// Variant tables (which (lpr, nv) pairs are compiled) -- used by the policy.
// lprc is the group class: lpr for lpr < 64, else 64.
bool fwd_variant_exists(int lprc, int nv, int wgs);
bool bwd_variant_exists(int lprc, int nv, int wgs);
bool fp8_variant_exists(int lprc, int nv, int wgs);

} // namespace rn

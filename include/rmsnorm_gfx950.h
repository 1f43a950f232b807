/*
 * rmsnorm_gfx950.h -- C ABI of the MI355X (gfx950) RMSNorm library.
 *
 * Operations, each one or two HIP kernels enqueued on the caller's stream:
 *   rmsnorm_fwd                   y = x * rstd * w, plus the fp32 rstd per row
 *   rmsnorm_bwd                   dx and the fp32 weight gradient dw in one pass
 *                                 over the rows (fixed-order, repeatable dw)
 *   add_rmsnorm_fp8_block_quant   residual add + RMSNorm + e4m3 1x128 block quant
 *   add_rmsnorm_fp8_quant         its variants: fp16 rows, e5m2 codes, or one
 *                                 given per-tensor scale
 *   rmsnorm_fwd_residual          training forward with a residual stream
 *   rmsnorm_bwd_residual          its backward (adds the residual-stream gradient)
 *   rmsnorm_fwd_heads             per-head RMSNorm (QK-norm) over (token, head) rows
 *
 * Conventions shared by every entry point
 *   - Every function is extern "C", never throws, never allocates device or
 *     host memory, never synchronizes the device and keeps no per-call state.
 *     The only global state is a once-per-device cache of device properties.
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     reads inputs and writes outputs only between enqueue and completion of
 *     its kernels on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream).  Results are visible to later work on that stream.
 *   - Matrices are row-major [T, H] with a row stride `ld*` counted in
 *     ELEMENTS (>= H).  Columns are contiguous.  Every matrix base pointer and
 *     row stride must be a multiple of 16 bytes, so each row splits into
 *     16-byte vectors; w must be 16-byte aligned, rstd, dw and block_scale
 *     4-byte aligned.  Buffers are compared by their byte extents: an output
 *     whose extent overlaps another buffer's is rejected (RN_ERR_ALIAS).
 *   - dtype codes: RN_F32 (IEEE binary32) or RN_BF16 (bfloat16, stored as
 *     its 16-bit pattern).  (x, w) pairs accepted: (f32, f32), (bf16, bf16),
 *     (bf16, f32).  dy and dx always share x's dtype; rstd and dw are fp32.
 *   - T >= 0; T == 0 returns RN_OK and enqueues nothing (except that
 *     the backwards then set dw to zero, the empty sum).  H >= 1, a multiple
 *     of 8 for bf16 rows and of 4 for f32 rows, and at most
 *       rmsnorm_fwd[_residual]       32768 (bf16 rows), 16384 (f32 rows)
 *       rmsnorm_bwd[_residual]       16384 (bf16 rows),  8192 (f32 rows)
 *       add_rmsnorm_fp8_block_quant  32768, a multiple of 128
 *     (RN_ERR_SHAPE beyond).
 *   - On any error the function returns a non-zero rn_status, enqueues
 *     nothing and touches no output.  Argument checks happen before any HIP
 *     call; a failed launch is reported as RN_ERR_LAUNCH.
 *   - Thread-safe.  Calls on one stream execute in order; calls on different
 *     streams that write the same buffers race (as any two kernels would).
 *
 * Sources of the operations (pages on the subject; titles and sections):
 *   [C] FlashInfer commit #5741 "cake_rmsnorm_train", quoted on the FlashInfer
 *       PR #4480 page: Summary; Design (Forward, Backward); API; Memory;
 *       Determinism.
 *   [F] FlashInfer PR #4480 "Add FusedAddRMSNormFP8BlockQuant": description
 *       (Kernel, API) and review thread (scale layout, e4m3 only, strides).
 *   [L] Liger-Kernel PR #1336 "perf(cutedsl): fused dX+dW backward +
 *       host-enqueue caching for RMSNorm": the fused single-pass dX+dW
 *       strip-reduction backward.
 *   [M] miles-ext-kernels PR #15 (re-vendoring the Cake RMSNorm packages):
 *       Summary and Accuracy, the per-element dw budget against an FP64 sum.
 *   [Q] FlashInfer PR #6332 (QKV projection + QK-RMSNorm + RoPE overlapped
 *       with the Ulysses head exchange): Description, operator math.
 */
#ifndef RMSNORM_GFX950_H
#define RMSNORM_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RN_OK = 0,
    RN_ERR_NULL = 1,        /* a required pointer is NULL                        */
    RN_ERR_SHAPE = 2,       /* T < 0, H out of range or not a vector multiple    */
    RN_ERR_DTYPE = 3,       /* unknown dtype code or unsupported (x, w) pair     */
    RN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                  */
    RN_ERR_STRIDE = 5,      /* a row stride < H, or not a 16-byte multiple       */
    RN_ERR_WORKSPACE = 6,   /* backward: workspace missing or too short          */
    RN_ERR_ALIAS = 7,       /* an output overlaps an input or another output     */
    RN_ERR_DEVICE = 8,      /* no current HIP device, or it is not gfx950        */
    RN_ERR_LAUNCH = 9       /* the kernel launch failed (hipGetLastError)        */
} rn_status;

typedef enum { RN_F32 = 0, RN_BF16 = 1, RN_F16 = 2 } rn_dtype;   /* RN_F16: the fp8 producer only */
typedef enum { RN_E4M3 = 0, RN_E5M2 = 1 } rn_fp8_format;

#define RN_MAX_H 32768
#define RN_HEADS_MAX_VECTORS 128   /* rmsnorm_fwd_heads: head_dim <= 1024 bf16 / 512 fp32 */

/* Human-readable name of a status code (static storage; never NULL). */
const char* rn_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int rn_version(void);

/*
 * RMSNorm forward  ([C] Summary and Design: Forward).
 *   rstd[r] = 1 / sqrt( (sum_j x[r,j]^2) / H + eps )        (fp32)
 *   y[r,j]  = round_dtype( x[r,j] * rstd[r] * w[j] )
 * The sum of squares and every product are fp32; the square root and the
 * divisions are IEEE (correctly rounded); y is rounded to x's dtype with
 * round-to-nearest-even.  rstd is what rmsnorm_bwd expects as its input.
 *   x     [T, ldx]  x_dtype        input
 *   w     [H]       w_dtype        input
 *   y     [T, ldy]  x_dtype        output (may not overlap x)
 *   rstd  [T]       fp32           output
 */
int rmsnorm_fwd(const void* x, int64_t ldx, int x_dtype,
                const void* w, int w_dtype,
                void* y, int64_t ldy, float* rstd,
                int64_t T, int64_t H, float eps, void* stream);

/*
 * Size in bytes of the workspace that rmsnorm_bwd needs for (T, H) on HIP
 * device `device`  ([C] API and Memory: the caller owns the backward's
 * workspace, sized by a query on (T, H, device) and reusable across T).
 * It holds fp32 partial sums, one per row strip and column (H rounded up to
 * a multiple of 16).  The value never decreases with T, so a workspace sized
 * for the largest T can be reused for every smaller T.  Returns 0 where no
 * workspace is used: T == 0, and rows that one strip walks alone (a few rows;
 * that launch writes dw directly), for bf16 and fp32 rows alike.  Returns
 * (size_t)-1 on invalid arguments or when the device cannot be queried.
 */
size_t rmsnorm_bwd_workspace_bytes(int64_t T, int64_t H, int device);

/*
 * RMSNorm backward: dx and dw in one pass over the rows
 * ([C] Design: Backward and Determinism; [L] fused dX+dW backward).
 *   xhat    = x * rstd
 *   c[r]    = (1/H) * sum_j dy[r,j] * w[j] * xhat[r,j]
 *   dx[r,j] = round_dtype( rstd[r] * (dy[r,j] * w[j] - c[r] * xhat[r,j]) )
 *   dw[j]   = sum_r dy[r,j] * x[r,j] * rstd[r]                (fp32 result)
 * rstd is the forward's stored fp32 value.  dw is OVERWRITTEN.  Each row
 * strip's dw partial is accumulated per column in FP64 from exact products
 * and rounded once to fp32 into `workspace`; a second kernel then sums the
 * strip partials of every column in a fixed order in FP64 and rounds once
 * more.  When the rows fit one strip (a few rows), that strip's partial is
 * dw itself: one kernel, no workspace.  dw is therefore bitwise identical
 * from call to call (the order depends only on T, H and the device's CU
 * count), and every element is within 1e-4 + 1e-4*|ref| of the FP64 sum
 * ([M] Summary).
 *   deterministic: both values run the fixed-order reduction above and give
 *     the same bits.  The non-deterministic form the pages describe (strip
 *     partials added into dw with fp32 atomics) was measured over the dw
 *     budget at T = 65536, H = 5120 (1.03x) and no faster, so it is not
 *     offered; the flag is kept for the interface.
 *   workspace: device memory of at least rmsnorm_bwd_workspace_bytes(T, H,
 *     device) bytes, 16-byte aligned, else RN_ERR_WORKSPACE.  May be NULL
 *     (with workspace_bytes 0) when that size is 0, whatever the flag.  Its
 *     content on entry does not matter and is garbage on return.
 *   dy [T, lddy] x_dtype; x [T, ldx] x_dtype; w [H] w_dtype; rstd [T] fp32
 *   dx [T, lddx] x_dtype output; dw [H] fp32 output.
 */
int rmsnorm_bwd(const void* dy, int64_t lddy,
                const void* x, int64_t ldx, int x_dtype,
                const void* w, int w_dtype,
                const float* rstd,
                void* dx, int64_t lddx, float* dw,
                int64_t T, int64_t H, int deterministic,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * rmsnorm_bwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same operation, arguments, kernels and bits as
 * rmsnorm_bwd; the strip partials live in a library-owned device array of
 * 8 MiB, one per device, kept until the process ends.  It holds the partials
 * of at most 256 row strips of up to 8192 columns: rows that one strip walks
 * (a few rows) are served at any H, more rows at H <= 8192 on a device of up
 * to 256 CUs; beyond that the call returns RN_ERR_WORKSPACE and enqueues
 * nothing.  Calls no allocating routine.  Every call on a device shares that
 * device's array: calls that overlap in time on one device (different
 * streams, or host threads without ordering) race on it and may return wrong
 * dw; calls ordered on one stream do not.  The array's content carries over
 * from call to call and is never read before it is written.
 */
int rmsnorm_bwd_noalloc(const void* dy, int64_t lddy,
                        const void* x, int64_t ldx, int x_dtype,
                        const void* w, int w_dtype,
                        const float* rstd,
                        void* dx, int64_t lddx, float* dw,
                        int64_t T, int64_t H, int deterministic, void* stream);

/*
 * Training forward with a residual stream  ([C] API and Design: Forward: the
 * forward that takes a residual returns h_new and normalises it).
 *   h[r,j]  = round_dtype( x[r,j] + u[r,j] )             written to h_out
 *   rstd[r] = 1 / sqrt( (sum_j h[r,j]^2) / H + eps )      (fp32)
 *   y[r,j]  = round_dtype( h[r,j] * rstd[r] * w[j] )
 * The sum is an fp32 addition rounded once to x's dtype (for two bf16 or two
 * fp32 inputs that is the correctly rounded sum); the rest is as in
 * rmsnorm_fwd, applied to h.  Same dtype pairs, limits and errors.
 *   x      [T, ldx]  x_dtype   input
 *   u      [T, ldu]  x_dtype   input (the residual stream)
 *   w      [H]       w_dtype   input
 *   y      [T, ldy]  x_dtype   output
 *   h_out  [T, ldh]  x_dtype   output; may be exactly x or exactly u (same
 *                              pointer and row stride: the update is then in
 *                              place), otherwise it may not overlap them
 *   rstd   [T]       fp32      output (what rmsnorm_bwd_residual expects)
 */
int rmsnorm_fwd_residual(const void* x, int64_t ldx, const void* u, int64_t ldu, int x_dtype,
                         const void* w, int w_dtype,
                         void* y, int64_t ldy, void* h_out, int64_t ldh, float* rstd,
                         int64_t T, int64_t H, float eps, void* stream);

/*
 * Training backward with a residual stream  ([C] API and Design: Backward:
 * the residual variant adds the gradient of the residual stream into the dx
 * it returns, so both inputs of the add receive the same gradient).
 * rmsnorm_bwd at x = the forward's h_out, plus
 *   dx[r,j] = round_dtype( rstd[r]*(dy[r,j]*w[j] - c[r]*xhat[r,j]) + g_residual[r,j] )
 * with the addition in fp32 before the one rounding.  dw does not depend on
 * g_residual.  Same workspace, limits and errors as rmsnorm_bwd.
 *   g_residual [T, ldgr] x_dtype  input; may be exactly dx (same pointer and
 *                                 row stride: dx then accumulates in place),
 *                                 otherwise it may not overlap dx
 */
int rmsnorm_bwd_residual(const void* dy, int64_t lddy,
                         const void* x, int64_t ldx, int x_dtype,
                         const void* w, int w_dtype,
                         const float* rstd,
                         const void* g_residual, int64_t ldgr,
                         void* dx, int64_t lddx, float* dw,
                         int64_t T, int64_t H, int deterministic,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-head RMSNorm, e.g. the QK-norm of attention  ([Q] Description,
 * operator math: an fp32 RMSNorm over each head's head_dim values with one
 * shared [head_dim] weight for all heads of Q, or of K).
 * Row (t, h), t < T, h < heads, is the head_dim values at
 *   x + t*ld_token + h*ld_head        (element offsets)
 * and is written to y + t*ldy_token + h*ldy_head; with r = t*heads + h,
 *   rstd[r] = 1 / sqrt( (sum_j row_j^2) / head_dim + eps )   (fp32)
 *   y_j     = round_dtype( row_j * rstd[r] * w[j] )
 * exactly as rmsnorm_fwd computes one row.  Q and K of a fused [T, (q+k+v)]
 * projection are two calls on column offsets of the same buffer.
 *   x, y  x_dtype; head_dim a multiple of 8 (bf16) / 4 (fp32) and at most
 *         RN_HEADS_MAX_VECTORS 16-byte vectors; ld_head >= head_dim when
 *         heads > 1, ld_token >= (heads-1)*ld_head + head_dim, both strides
 *         16-byte multiples (else RN_ERR_STRIDE); 1 <= heads <= 65535 and
 *         T*heads < 2^31 (else RN_ERR_SHAPE).
 *   y     may be exactly x with the same strides (in place); otherwise the
 *         byte extents of x and y may not overlap (RN_ERR_ALIAS).
 *   w     [head_dim] w_dtype.
 *   rstd  [T*heads] fp32 output, token-major; may be NULL (not stored).
 */
int rmsnorm_fwd_heads(const void* x, int64_t ld_token, int64_t ld_head, int x_dtype,
                      const void* w, int w_dtype,
                      void* y, int64_t ldy_token, int64_t ldy_head, float* rstd,
                      int64_t T, int64_t heads, int64_t head_dim, float eps, void* stream);

/*
 * Fused residual add + RMSNorm + FP8 e4m3 1x128 block quant
 * ([F] description: Kernel and API; review thread on the scale layout).
 * bf16 only; H a multiple of 128.  Per row r:
 *   h[r,j]      = bf16( x[r,j] + residual[r,j] )     written back to residual
 *   rstd        = 1 / sqrt( (sum_j h[r,j]^2) / H + eps )   (fp32, not stored)
 *   n[r,j]      = bf16( h[r,j] * rstd * w[j] )        written to normed_out
 *   per block k (columns 128k .. 128k+127):
 *     a         = max_j |n[r,j]|                      (exact)
 *     s         = a / 448.0f                          (IEEE fp32 division)
 *     block_scale[k * scale_ld + r] = s
 *     out[r,j]  = e4m3fn( n[r,j] / s )   IEEE fp32 quotient, rounded to
 *                 nearest even onto E4M3FN, saturating at +-448, sign kept;
 *                 an all-zero block has s = 0 and codes 0x00.
 * The codes are therefore exactly a re-quantisation of normed_out.
 *   x           [T, ldx]  bf16   input
 *   residual    [T, ldr]  bf16   input and output (in place; the only
 *                                buffer that may be both)
 *   w           [H]       bf16   input
 *   out         [T, ldo]  uint8  e4m3fn codes, output (ldo in bytes, %16 == 0)
 *   block_scale [H/128, scale_ld] fp32 output, row index fastest
 *               (column-major (H/128, round_up(T,4)) when scale_ld is
 *               round_up(T,4)); scale_ld >= T and scale_ld % 4 == 0; entries
 *               for rows T .. scale_ld-1 are not written.
 *   normed_out  [T, ldn]  bf16   output
 */
int add_rmsnorm_fp8_block_quant(const void* x, int64_t ldx,
                                void* residual, int64_t ldr,
                                const void* w,
                                uint8_t* out, int64_t ldo,
                                float* block_scale, int64_t scale_ld,
                                void* normed_out, int64_t ldn,
                                int64_t T, int64_t H, float eps, void* stream);

/*
 * Producer variants  ([F] description: the block-scaled sibling of the
 * per-tensor FusedAddRMSNormQuant, its tests over fp16 and bf16 inputs;
 * review thread: the bound 448 belongs to e4m3 and follows the output type).
 * As add_rmsnorm_fp8_block_quant, generalised:
 *   dtype       RN_BF16 or RN_F16: x, residual, w and normed_out all have it;
 *               h and n are rounded to it (nearest even).
 *   out_format  RN_E4M3 (MAX = 448) or RN_E5M2 (MAX = 57344).
 *   exactly one of
 *     block_scale   block-scale form, as in add_rmsnorm_fp8_block_quant with
 *                   s = a / MAX;
 *     tensor_scale  per-tensor form: a DEVICE pointer to one fp32 scale s used
 *                   for every element; codes = fp8(clamp(n / s, -MAX, MAX))
 *                   with the IEEE fp32 quotient rounded to nearest even; no
 *                   scales are written.  s must be a positive number (codes
 *                   are 0x00 otherwise).  Both non-NULL or both NULL:
 *                   RN_ERR_NULL.
 *   normed_out  may be NULL (not written).
 * With dtype RN_BF16, out_format RN_E4M3 and block_scale this computes what
 * add_rmsnorm_fp8_block_quant computes, bit for bit.  Same limits and errors.
 */
int add_rmsnorm_fp8_quant(const void* x, int64_t ldx,
                          void* residual, int64_t ldr,
                          const void* w, int dtype,
                          uint8_t* out, int64_t ldo, int out_format,
                          float* block_scale, int64_t scale_ld,
                          const float* tensor_scale,
                          void* normed_out, int64_t ldn,
                          int64_t T, int64_t H, float eps, void* stream);

/*
 * Host-only launch policy query (no HIP call; usable without a GPU).
 * op: 0 = forward (also per-head, with T = tokens * heads and H = head_dim),
 * 1 = backward, 2 = fused fp8 producer, 3 = forward with a residual stream,
 * 4 = backward with a residual stream.
 * Fills out[0..6] = { lanes per row, 16-byte vectors per lane, threads per
 * work-group, work-groups (row chunks), rows per work-group pass, kernel id,
 * flags (bit 0: non-temporal streaming loads/stores, bit 1: interleaved row
 * walk, bits 4-6: row buffers in the ring, 0 meaning the default two) }
 * for a device with `cu_count` compute units.  Returns an rn_status.
 */
int rn_query_policy(int op, int64_t T, int64_t H, int x_dtype, int w_dtype,
                    int cu_count, int32_t* out);

/* Workspace bytes for a device with `cu_count` CUs (host-only twin of
 * rmsnorm_bwd_workspace_bytes). */
size_t rn_bwd_workspace_bytes_for(int64_t T, int64_t H, int cu_count);

/*
 * Self-test hooks for the fp8 producer's quantisation step (diagnostics; the
 * test suite calls them on a GPU).
 * rn_selftest_quant: for every bf16 block maximum a with bit pattern in
 *   [a_lo, a_hi] (1 .. 0x7f7f) and every bf16 n with |n| <= a (both signs),
 *   compares the codes the producer kernel computes for n with scale
 *   s = a/448 against e4m3(n / s) with the IEEE fp32 division; adds the
 *   number of mismatching 8-value chunks to *d_mismatches and lowers
 *   *d_first_bad to (a << 16 | n-magnitude) of the first failure.  Both are
 *   device pointers the caller initialises.  Returns 0, 2 (bad range) or 9.
 * rn_selftest_cvt_e4m3 / _e5m2: d_out[i] = e4m3 / e5m2 code of fp32 d_in[i]
 *   (i < n), made by the same conversion instruction the producer uses.
 *   Returns 0, 1 or 9.
 * rn_selftest_quotient: the producer's quotient n / s against the IEEE fp32
 *   division: the fp8 codes of the two for every pair, and the quotients bit
 *   for bit wherever |n| >= 2^-100 and the IEEE quotient is a normal number
 *   below 2 * MAX.
 *   d_scales == NULL: block-scale form, for every amax pattern of `dtype` in
 *   [a_lo, a_hi] (s = amax / MAX) and every n of that dtype with |n| <= amax;
 *   otherwise per-tensor form, for each of the n_scales (<= 65535) device
 *   scales and every finite n of the dtype.  Counts mismatches into
 *   *d_mismatches and lowers *d_first_bad as rn_selftest_quant does.
 *   Returns 0, 1, 2 (bad range), 3 (bad dtype or format) or 9.
 */
int rn_selftest_quant(uint32_t a_lo, uint32_t a_hi, unsigned long long* d_mismatches,
                      uint32_t* d_first_bad, void* stream);
int rn_selftest_cvt_e4m3(const float* d_in, uint8_t* d_out, int64_t n, void* stream);
int rn_selftest_cvt_e5m2(const float* d_in, uint8_t* d_out, int64_t n, void* stream);
int rn_selftest_quotient(int dtype, int out_format, uint32_t a_lo, uint32_t a_hi, const float* d_scales,
                         int64_t n_scales, unsigned long long* d_mismatches, uint32_t* d_first_bad,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_GFX950_H */

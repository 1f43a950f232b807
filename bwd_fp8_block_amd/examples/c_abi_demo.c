/*
 * c_abi_demo.c -- the RMSNorm library called from plain C through its C ABI.
 *
 * Host-generated bf16 inputs (standard normal rows, weights 1 + 0.1 N(0,1)),
 * device buffers from hipMalloc and one HIP stream; then, in stream order,
 *   rmsnorm_fwd                  y, rstd
 *   rmsnorm_bwd                  dx, dw (workspace sized by the library's query)
 *   add_rmsnorm_fp8_block_quant  residual (in place), e4m3 codes, block scales,
 *                                bf16 normed
 * and every input and output is written to a file, so that a checker can
 * compare them with a reference.  No Python and no PyTorch are involved.
 *
 * usage: c_abi_demo OUT_FILE [T H]     (H a multiple of 128, default 257 x 4096)
 *
 * File layout (little endian): the 8-byte tag "RNDEMO01", then int64 T, H and
 * scale_ld, then the arrays in this order, each row-major and dense:
 *   x, w, dy, residual_in          uint16 bf16 bits   [T,H] [H] [T,H] [T,H]
 *   y                              uint16 bf16 bits   [T,H]
 *   rstd                           float32            [T]
 *   dx                             uint16 bf16 bits   [T,H]
 *   dw                             float32            [H]
 *   residual_out                   uint16 bf16 bits   [T,H]
 *   codes                          uint8 e4m3fn       [T,H]
 *   block_scale                    float32            [H/128, scale_ld]
 *   normed                         uint16 bf16 bits   [T,H]
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/rmsnorm_gfx950.h"

#define HIP_OK(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "c_abi_demo: %s failed: %s\n", #call, hipGetErrorString(e_));     \
            return 1;                                                                         \
        }                                                                                     \
    } while (0)

#define RN_OK_(call)                                                                          \
    do {                                                                                      \
        int s_ = (call);                                                                      \
        if (s_ != RN_OK) {                                                                    \
            fprintf(stderr, "c_abi_demo: %s returned %s\n", #call, rn_status_string(s_));     \
            return 1;                                                                         \
        }                                                                                     \
    } while (0)

/* xorshift64* and Box-Muller: a fixed, portable input stream. */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform01(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static double normal01(void)
{
    double u = uniform01(), v = uniform01();
    if (u < 1e-300) u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static int write_all(FILE* f, const void* p, size_t n)
{
    return fwrite(p, 1, n, f) == n ? 0 : 1;
}

int main(int argc, char** argv)
{
    if (argc != 2 && argc != 4) {
        fprintf(stderr, "usage: c_abi_demo OUT_FILE [T H]\n");
        return 2;
    }
    const int64_t T = argc == 4 ? atoll(argv[2]) : 257;
    const int64_t H = argc == 4 ? atoll(argv[3]) : 4096;
    if (T < 1 || H < 128 || H % 128 != 0 || H > 16384) {
        fprintf(stderr, "c_abi_demo: T >= 1 and H a multiple of 128 up to 16384\n");
        return 2;
    }
    const int64_t ld = (T + 3) / 4 * 4;             /* block-scale row stride */
    const size_t n = (size_t)(T * H), nb = n * 2, nsc = (size_t)(H / 128 * ld);
    const float eps = 1e-6f;

    uint16_t *x = malloc(nb), *w = malloc((size_t)H * 2), *dy = malloc(nb), *res = malloc(nb);
    uint16_t *y = malloc(nb), *dx = malloc(nb), *res_out = malloc(nb), *normed = malloc(nb);
    float *rstd = malloc((size_t)T * 4), *dw = malloc((size_t)H * 4), *scale = malloc(nsc * 4);
    uint8_t* codes = malloc(n);
    if (!x || !w || !dy || !res || !y || !dx || !res_out || !normed || !rstd || !dw || !scale || !codes) {
        fprintf(stderr, "c_abi_demo: out of host memory\n");
        return 1;
    }
    for (size_t i = 0; i < n; ++i) x[i] = to_bf16((float)normal01());
    for (int64_t j = 0; j < H; ++j) w[j] = to_bf16((float)(1.0 + 0.1 * normal01()));
    for (size_t i = 0; i < n; ++i) dy[i] = to_bf16((float)normal01());
    for (size_t i = 0; i < n; ++i) res[i] = to_bf16((float)normal01());

    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void *x_d, *w_d, *dy_d, *r_d, *y_d, *dx_d, *n_d, *rstd_d, *dw_d, *sc_d, *o_d, *ws_d = NULL;
    HIP_OK(hipMalloc(&x_d, nb));
    HIP_OK(hipMalloc(&w_d, (size_t)H * 2));
    HIP_OK(hipMalloc(&dy_d, nb));
    HIP_OK(hipMalloc(&r_d, nb));
    HIP_OK(hipMalloc(&y_d, nb));
    HIP_OK(hipMalloc(&dx_d, nb));
    HIP_OK(hipMalloc(&n_d, nb));
    HIP_OK(hipMalloc(&rstd_d, (size_t)T * 4));
    HIP_OK(hipMalloc(&dw_d, (size_t)H * 4));
    HIP_OK(hipMalloc(&sc_d, nsc * 4));
    HIP_OK(hipMalloc(&o_d, n));
    HIP_OK(hipMemcpy(x_d, x, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w_d, w, (size_t)H * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy_d, dy, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(r_d, res, nb, hipMemcpyHostToDevice));

    /* forward: y and the fp32 rstd the backward takes */
    RN_OK_(rmsnorm_fwd(x_d, H, RN_BF16, w_d, RN_BF16, y_d, H, (float*)rstd_d, T, H, eps, s));

    /* backward: the caller owns the workspace, sized by the library */
    const size_t ws = rmsnorm_bwd_workspace_bytes(T, H, dev);
    if (ws == (size_t)-1) {
        fprintf(stderr, "c_abi_demo: rmsnorm_bwd_workspace_bytes rejected (T, H)\n");
        return 1;
    }
    if (ws) HIP_OK(hipMalloc(&ws_d, ws));
    RN_OK_(rmsnorm_bwd(dy_d, H, x_d, H, RN_BF16, w_d, RN_BF16, (const float*)rstd_d, dx_d, H, (float*)dw_d, T, H,
                       1, ws_d, ws, s));

    /* fused residual add + RMSNorm + FP8 1x128 block quant (residual updated in place) */
    RN_OK_(add_rmsnorm_fp8_block_quant(x_d, H, r_d, H, w_d, (uint8_t*)o_d, H, (float*)sc_d, ld, n_d, H, T, H, eps,
                                       s));
    HIP_OK(hipStreamSynchronize(s));

    HIP_OK(hipMemcpy(y, y_d, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rstd, rstd_d, (size_t)T * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dx, dx_d, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dw, dw_d, (size_t)H * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(res_out, r_d, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(codes, o_d, n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(scale, sc_d, nsc * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(normed, n_d, nb, hipMemcpyDeviceToHost));

    FILE* f = fopen(argv[1], "wb");
    if (!f) {
        fprintf(stderr, "c_abi_demo: cannot open %s\n", argv[1]);
        return 1;
    }
    const int64_t hdr[3] = {T, H, ld};
    int bad = write_all(f, "RNDEMO01", 8) | write_all(f, hdr, sizeof hdr);
    bad |= write_all(f, x, nb) | write_all(f, w, (size_t)H * 2) | write_all(f, dy, nb) | write_all(f, res, nb);
    bad |= write_all(f, y, nb) | write_all(f, rstd, (size_t)T * 4) | write_all(f, dx, nb);
    bad |= write_all(f, dw, (size_t)H * 4) | write_all(f, res_out, nb) | write_all(f, codes, n);
    bad |= write_all(f, scale, nsc * 4) | write_all(f, normed, nb);
    bad |= fclose(f) != 0;
    if (bad) {
        fprintf(stderr, "c_abi_demo: writing %s failed\n", argv[1]);
        return 1;
    }

    HIP_OK(hipFree(x_d));
    HIP_OK(hipFree(w_d));
    HIP_OK(hipFree(dy_d));
    HIP_OK(hipFree(r_d));
    HIP_OK(hipFree(y_d));
    HIP_OK(hipFree(dx_d));
    HIP_OK(hipFree(n_d));
    HIP_OK(hipFree(rstd_d));
    HIP_OK(hipFree(dw_d));
    HIP_OK(hipFree(sc_d));
    HIP_OK(hipFree(o_d));
    if (ws_d) HIP_OK(hipFree(ws_d));
    HIP_OK(hipStreamDestroy(s));
    printf("c_abi_demo: T=%lld H=%lld, library version %d, workspace %zu bytes: ok\n", (long long)T, (long long)H,
           rn_version(), ws);
    free(x); free(w); free(dy); free(res); free(y); free(dx); free(res_out); free(normed);
    free(rstd); free(dw); free(scale); free(codes);
    return 0;
}

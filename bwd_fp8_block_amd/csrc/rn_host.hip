// rn_host.hip -- C ABI of the gfx950 RMSNorm library: argument validation,
// launch policy and enqueue.  Never allocates, never synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/rmsnorm_gfx950.h"
#include "rn_internal.h"

using rn::Policy;

// ---------------------------------------------------------------------------
// Library-owned scratch for rmsnorm_bwd_noalloc: the dw strip partials of a
// backward launch, for callers that cannot allocate device memory.  Every
// device that loads the library holds its own copy of this array until the
// process ends; host code reaches a device's copy only through the address
// hipGetSymbolAddress returns with that device current (the array's name on
// the host is a stand-in, not a device address).  256 strips x 8192 columns
// of fp32: 8 MiB.
// ---------------------------------------------------------------------------
constexpr size_t kScratchFloats = (size_t)256 * 8192;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

// ---------------------------------------------------------------------------
// Per-device property cache (the only global state).
// ---------------------------------------------------------------------------
struct DevInfo {
    std::atomic<int> state{0};   // 0 unknown, 1 ok, 2 not gfx950 / error
    int cu = 0;
};
constexpr int kMaxDev = 64;
DevInfo g_dev[kMaxDev];
std::mutex g_dev_mu;

int device_cu(int dev, int* cu)
{
    if (dev < 0 || dev >= kMaxDev) return RN_ERR_DEVICE;
    DevInfo& d = g_dev[dev];
    int st = d.state.load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        st = d.state.load(std::memory_order_relaxed);
        if (st == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
                st = 2;
            } else {
                st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.multiProcessorCount > 0) ? 1 : 2;
                d.cu = prop.multiProcessorCount;
            }
            d.state.store(st, std::memory_order_release);
        }
    }
    if (st != 1) return RN_ERR_DEVICE;
    *cu = d.cu;
    return RN_OK;
}

int current_device_cu(int* cu)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RN_ERR_DEVICE;
    return device_cu(dev, cu);
}

// The current device's copy of `scratch`: its address is taken once per
// device, with that device current, and kept.
struct ScratchSlot {
    std::atomic<int> state{0};   // 0 unknown, 1 ok, 2 failed
    float* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDev];

int current_scratch(float** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return RN_ERR_DEVICE;
    ScratchSlot& sl = g_scratch[dev];
    int st = sl.state.load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        st = sl.state.load(std::memory_order_relaxed);
        if (st == 0) {
            void* p = nullptr;
            st = (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) ? 1 : 2;
            sl.ptr = static_cast<float*>(p);
            sl.state.store(st, std::memory_order_release);
        }
    }
    if (st != 1) return RN_ERR_DEVICE;
    *out = sl.ptr;
    return RN_OK;
}

// ---------------------------------------------------------------------------
// Optional policy override for tuning sweeps, read once: RN_POLICY_FWD,
// RN_POLICY_BWD, RN_POLICY_FP8 = "lpr,nv,wgs,grid[,flags]" (0 keeps the
// default; flags -1 or absent keeps the default).
// ---------------------------------------------------------------------------
struct Override { int lpr = 0, nv = 0, wgs = 0; long long grid = 0; int flags = -1; };
Override g_ovr[3];
std::once_flag g_ovr_once;
bool g_log = false;

void read_overrides()
{
    const char* names[3] = {"RN_POLICY_FWD", "RN_POLICY_BWD", "RN_POLICY_FP8"};
    for (int k = 0; k < 3; ++k) {
        const char* v = std::getenv(names[k]);
        if (v)
            std::sscanf(v, "%d,%d,%d,%lld,%d", &g_ovr[k].lpr, &g_ovr[k].nv, &g_ovr[k].wgs, &g_ovr[k].grid,
                        &g_ovr[k].flags);
    }
    const char* l = std::getenv("RN_LOG");
    g_log = l && l[0] == '1';
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Streaming (non-temporal) loads and stores by default: every byte of the
// row tensors is touched exactly once per call.
constexpr int RN_FLAG_NT_DEFAULT = rn::RN_FLAG_NT;

// Threads per work-group for a row-group width: as many whole groups as fit
// in `cap` threads.
int wgs_for(int lpr, int cap) { return lpr >= cap ? lpr : lpr * (cap / lpr); }

int elems_per_chunk(int dt) { return dt == RN_BF16 ? 8 : 4; }
int elem_bytes(int dt) { return dt == RN_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Launch policies (pure functions of the shape and the CU count).
// ---------------------------------------------------------------------------

// Forward.  Rows split over two wavefronts with at most 4-8 vectors of 16
// bytes per lane, walked as one interleaved window.  Short rows (up to 128
// vectors) take sub-wavefront groups of 8 to 32 lanes with up to 4 vectors
// per lane; very long rows more wavefronts.  Work-groups per CU, measured on
// MI355X: for rows of 2-16 KiB four while T is at most 48 rows per CU (T =
// 8192: 0.95-0.97 of a same-traffic streaming copy) and two beyond (T =
// 16384 .. 65536: 0.94-0.97, where four fall to 0.87-0.94); for short rows
// (H = 128 .. 1024, T = 65536 .. 2^21) four up to 512 rows per CU (0.96-1.0),
// beyond that eight for 8-lane groups and two for 16/32-lane groups
// (0.85-0.95).
int fwd_per_cu(int64_t T, int cu, const Policy& p)
{
    const bool long_run = T > 512 * (int64_t)cu;
    if (p.lpr <= 8) return long_run ? 8 : 4;
    if (p.lpr < 64) return long_run ? 2 : 4;
    if (p.nv <= 4) return T <= 48 * (int64_t)cu ? 4 : 2;
    return 2;
}

int policy_fwd(int64_t T, int64_t H, int x_dtype, int cu, Policy* p)
{
    const int nch = (int)(H / elems_per_chunk(x_dtype));
    if (nch <= 8)         { p->lpr = 8; p->nv = 1; }
    else if (nch <= 16)   { p->lpr = 8; p->nv = 2; }
    else if (nch <= 32)   { p->lpr = 8; p->nv = 4; }
    else if (nch <= 64)   { p->lpr = 16; p->nv = 4; }
    else if (nch <= 128)  { p->lpr = 32; p->nv = 4; }
    else if (nch <= 256)  { p->lpr = 64; p->nv = (int)ceil_div(nch, 64); }
    else if (nch <= 1024) { p->lpr = 128; p->nv = (int)ceil_div(nch, 128); }
    else                  { p->lpr = 64 * (int)ceil_div(nch, 64 * 8); p->nv = (int)ceil_div(nch, p->lpr); }
    if (p->lpr > 512) return RN_ERR_SHAPE;
    // Rows of 5-8 vectors per 128-lane group (H = 4104 .. 8192 bf16): four groups
    // to a 512-thread work-group, one per CU once each CU's share of the tensor is
    // at least 13312 chunks, two below that.  Measured on MI355X against two
    // 256-thread work-groups per CU: T = 65536, H = 5120 / 6144 / 7168 219 / 272 /
    // 320 us vs 232 / 298 / 363; T = 16384 6-10% faster, T = 8192 1-5%; T = 4096,
    // H = 5120 / 6144 14.6 / 17.4 us with two per CU (15.5 / 18.2 before).
    const bool wide = p->lpr == 128 && p->nv >= 5;
    p->wgs = wide ? 512 : wgs_for(p->lpr, 256);
    p->gpw = p->wgs / p->lpr;
    const int64_t per_cu = wide ? (T * nch >= 13312 * (int64_t)cu ? 1 : 2) : fwd_per_cu(T, cu, *p);
    int64_t g = ceil_div(T, p->gpw);
    if (g > (int64_t)cu * per_cu) g = (int64_t)cu * per_cu;
    p->grid = g < 1 ? 1 : g;
    p->kernel = 0;
    p->flags = RN_FLAG_NT_DEFAULT | rn::RN_FLAG_ILV;
    return RN_OK;
}

// The residual form reads two rows (x, u) and writes two (y, h_new) for every
// row of the plain forward: same row geometry, half the work-groups.
// Measured on MI355X: two per CU up to 64 rows per CU (T = 8192, H = 2048 ..
// 4096: 0.95-0.97 of a same-traffic copy), one beyond (T = 32768 .. 65536:
// 0.91-0.95) and for rows of more than four vectors per lane (T = 8192,
// H = 5120 / 7168: 0.89 / 0.93).
int policy_fwd_residual(int64_t T, int64_t H, int x_dtype, int cu, Policy* p)
{
    const int st = policy_fwd(T, H, x_dtype, cu, p);
    if (st != RN_OK) return st;
    if (p->lpr == 128 && p->wgs == 512) {        // keeps two 128-lane groups per work-group
        p->wgs = 256;
        p->gpw = 2;
    }
    const int64_t per_cu = p->lpr < 64 ? std::max(1, fwd_per_cu(T, cu, *p) / 2)
                         : (p->nv <= 4 && T <= 64 * (int64_t)cu) ? 2 : 1;
    int64_t g = ceil_div(T, p->gpw);
    if (g > (int64_t)cu * per_cu) g = (int64_t)cu * per_cu;
    p->grid = g < 1 ? 1 : g;
    p->kernel = 3;
    return RN_OK;
}

// Backward: few vectors per lane so that the FP64 dw accumulators stay in
// registers; one work-group (one row strip) per CU.
//   Few rows: one vector per lane (two beyond 1024 chunks) in 1024-thread
//   groups, and a single strip that writes dw itself when each row group walks
//   at most two rows (four for rows of at most 64 vectors): measured on MI355X
//   at 4.3-5.8 us against 6.5-7.3 us for two launches.  The strip count then
//   depends only on T and H, so the bits of dw do not depend on the device's
//   CU count.
//   Streaming: rows of up to 512 chunks take one vector per lane (16- and
//   32-lane groups for rows of up to 16 / 32 chunks) in 512-thread groups;
//   rows of 513 .. 1024 chunks two vectors per lane in one group of at most 512
//   lanes; both with three row buffers (two rows of loads in flight per row
//   group).  Rows wider than 1024 chunks take two vectors per lane in one group
//   of more than 512 lanes with two buffers.  Measured on MI355X:
//   - against 1024-thread groups with two buffers: bf16 T=8192 H=4096 39.5 us
//     vs 41.3, H=2048 T=58497 118 vs 125, H=5120 T=65536 353 vs 403; short rows
//     at T=65536: H=128 15.7 vs 18.1, H=256 22.9 vs 24.6;
//   - wide rows against one vector per lane in one group of up to 1024 lanes:
//     H = 5120 / 6144 / 7168 / 8192 at T = 8192 47.9 / 53.3 / 62.1 / 70.4 us
//     vs 48.0 / 58.1 / 67.4 / 75.9, at T = 4096 28.6 / 31.6 / 35.8 / 38.9 vs
//     29.2 / 34.6 / 40.2 / 45.9, T = 65536, H = 5120 (fp32 weight) 319 vs 341;
//     two such groups per strip were 3x slower.
int policy_bwd(int64_t T, int64_t H, int x_dtype, int cu, Policy* p)
{
    const int nch = (int)(H / elems_per_chunk(x_dtype));
    if (nch <= 16)        { p->lpr = 16; p->nv = 1; }
    else if (nch <= 32)   { p->lpr = 32; p->nv = 1; }
    else if (nch <= 1024) { p->lpr = 64 * (int)ceil_div(nch, 64); p->nv = 1; }
    else                  { p->lpr = 64 * (int)ceil_div(nch, 128); p->nv = 2; }
    if (p->lpr > 1024) return RN_ERR_SHAPE;
    p->kernel = 1;
    p->flags = RN_FLAG_NT_DEFAULT | rn::RN_FLAG_ILV;
    p->wgs = wgs_for(p->lpr, 1024);
    p->gpw = p->wgs / p->lpr;
    const int64_t iters = ceil_div(T, p->gpw);
    if (iters <= 2 || (iters <= 4 && nch <= 64)) {
        p->grid = 1;
        return RN_OK;
    }
    if (p->nv == 1) {
        if (nch > 512) {                         // wide rows: two vectors per lane, one group of <= 512 lanes
            p->lpr = 64 * (int)ceil_div(nch, 128);
            p->nv = 2;
        }
        p->wgs = wgs_for(p->lpr, 512);
        p->gpw = p->wgs / p->lpr;
        p->flags |= 3 << 4;                      // three row buffers
    }
    int64_t g = ceil_div(T, p->gpw);
    if (g > (int64_t)cu) g = cu;
    p->grid = g < 1 ? 1 : g;
    return RN_OK;
}

// True when the rows of a backward fit one strip's walk: the policy then
// launches a single work-group that writes dw itself, whatever the CU count,
// and no workspace is used.  (With any number of CUs the grid of the other
// case has at least min(3, cu) strips.)
bool bwd_one_strip(int64_t T, int64_t H, int x_dtype)
{
    Policy p{};
    if (policy_bwd(T, H, x_dtype, 1 << 20, &p) != RN_OK) return false;
    return p.grid == 1;
}

// Backward with a residual stream: as the plain backward, except that
//   - groups wider than 512 lanes keep two row buffers: the extra g_residual
//     buffer of a third does not fit the registers of a 1024-thread group
//     (measured on MI355X: bf16 T = 8192, H = 7168 with one vector per lane,
//     105 us with three buffers against 92 us with two).  The wide-row form of
//     the plain backward (two vectors per lane, one group of at most 512 lanes,
//     three buffers) measured T = 8192 / 65536, H = 5120 63.3 / 484 us against
//     70.6 / 524 with one vector per lane, and H = 7168 within 3% either way
//     (T = 4096 .. 8192);
//   - where the plain backward streams with three buffers, the residual one,
//     which loads a third row for every row, streams with two in the steady
//     form (one row of loads in flight), measured faster or equal at every
//     shape tried on MI355X: bf16 T = 8192, H = 4096 46.3 against 47.4 us;
//     T = 58497, H = 2048 with fp32 weight 156.6 against 162.4; T = 32768,
//     H = 5120 231.7 against 239.5; 1-4% less over H = 256 .. 7168,
//     T = 1024 .. 32768; T = 65536, H = 4096 375.7 against 374.6.
int policy_bwd_residual(int64_t T, int64_t H, int x_dtype, int cu, Policy* p)
{
    const int st = policy_bwd(T, H, x_dtype, cu, p);
    if (st != RN_OK) return st;
    if (p->wgs > 512) p->flags &= ~(7 << 4);
    else if (((p->flags >> 4) & 7) == 3) p->flags = (p->flags & ~(7 << 4)) | (2 << 4) | rn::RN_FLAG_STEADY;
    return RN_OK;
}

// Fused fp8 producer: a 1x128 block is 16 lanes, so groups are 16, 32 or a
// multiple of 64 lanes.  Rows of 129 .. 896 chunks (H = 1152 .. 7168) take
// 128-lane groups with up to 7 vectors per lane, four groups to a 512-thread
// work-group; one such work-group per CU once each CU's share of the tensor is
// at least 10240 chunks, two below that.  Measured on MI355X against two
// 256-thread work-groups per CU (lpr 128 up to H = 4096, lpr 256 beyond), for
// the block-scale, per-tensor and fp16/e5m2 forms: T = 32768, H = 4096 203 /
// 209 / 199 us vs 221 / 219 / 225; T = 32768, H = 2048 102 vs 111 (block);
// T = 4096, H = 7168 47.6 / 52.2 / 49.2 vs 50.4 / 52.1 / 51.3; T = 8192,
// H = 2048 / 3072 2-8% faster; H = 5120 and 6144 3-9% faster.  Rows of 4
// vectors switch only from 32768 chunks per CU: at T = 8192, H = 4096 the
// block-scale form ties (53.4 vs 53.2 us) and the per-tensor form is slower
// (57.5 vs 54.6).  Rows of 897 .. 1024 chunks take 256-lane groups with 4
// vectors per lane, two to a 512-thread work-group, two such work-groups per
// CU below 32768 chunks per CU and one from there: H = 8192, T = 16384 / 65536
// 204 / 823 us against 222 / 926 with one group per 256-thread work-group
// (two per CU), T = 4096 54.1 against 54.7; 128 lanes x 8 took 871 us at
// T = 65536.
int policy_fp8(int64_t T, int64_t H, int cu, Policy* p)
{
    const int nch = (int)(H / 8);
    if (nch <= 16)        { p->lpr = 16; p->nv = 1; }
    else if (nch <= 32)   { p->lpr = 32; p->nv = 1; }
    else if (nch <= 64)   { p->lpr = 64; p->nv = 1; }
    else if (nch <= 896)  { p->lpr = 128; p->nv = (int)ceil_div(nch, 128); }
    else if (nch <= 1024) { p->lpr = 256; p->nv = (int)ceil_div(nch, 256); }
    else                  { p->lpr = 64 * (int)ceil_div(nch, 64 * 8); p->nv = (int)ceil_div(nch, p->lpr); }
    if (p->lpr > 512) return RN_ERR_SHAPE;
    const int64_t cpc = T * nch / cu;           // chunks of one row tensor per CU
    bool wide_groups = false;                   // 512-thread work-groups
    int64_t per_cu = 2;
    if (p->lpr == 128 && p->nv >= 2 && p->nv != 4) {
        wide_groups = true;
        per_cu = cpc >= 10240 ? 1 : 2;
    } else if (p->lpr == 128 && p->nv == 4) {
        wide_groups = cpc >= 32768;
        per_cu = wide_groups ? 1 : 2;
    } else if (p->lpr == 256 && p->nv == 4) {
        wide_groups = true;
        per_cu = cpc >= 32768 ? 1 : 2;
    }
    p->wgs = wide_groups ? 512 : wgs_for(p->lpr, 256);
    p->gpw = p->wgs / p->lpr;
    int64_t g = ceil_div(T, p->gpw);
    if (g > (int64_t)cu * per_cu) g = (int64_t)cu * per_cu;
    p->grid = g < 1 ? 1 : g;
    p->kernel = 2;
    p->flags = RN_FLAG_NT_DEFAULT | rn::RN_FLAG_ILV;
    return RN_OK;
}

// Apply a tuning override; refuse anything that no compiled variant serves or
// that breaks the geometry invariants (wgs a multiple of lpr, lpr % 64 == 0
// beyond 32 lanes, 16-lane blocks for the fp8 kernel).
void apply_override(int op, int64_t T, int nch, Policy* p)
{
    std::call_once(g_ovr_once, read_overrides);
    const Override& o = g_ovr[op];
    if (!o.lpr && !o.nv && !o.wgs && !o.grid && o.flags < 0) return;
    Policy q = *p;
    if (o.flags >= 0) q.flags = o.flags;
    if (o.lpr) q.lpr = o.lpr;
    if (o.nv) q.nv = o.nv;
    if (o.wgs) q.wgs = o.wgs;
    else q.wgs = wgs_for(q.lpr, op == 1 ? 1024 : 256);
    if (q.lpr <= 0 || q.wgs <= 0 || q.wgs > 1024 || q.wgs % q.lpr != 0) return;
    if (op == 2 && q.lpr % 16 != 0) return;
    if (q.lpr != 16 && q.lpr != 32 && q.lpr % 64 != 0 && !(op == 0 && (q.lpr == 4 || q.lpr == 8))) return;
    if ((int64_t)q.lpr * q.nv < nch) return;
    q.gpw = q.wgs / q.lpr;
    const int lprc = q.lpr < 64 ? q.lpr : 64;
    const bool ok = op == 0 ? rn::fwd_variant_exists(lprc, q.nv, q.wgs)
                  : op == 1 ? rn::bwd_variant_exists(lprc, q.nv, q.wgs)
                            : rn::fp8_variant_exists(lprc, q.nv, q.wgs);
    if (!ok) return;
    if (o.grid) q.grid = std::max<int64_t>(1, std::min<int64_t>(o.grid, ceil_div(T, q.gpw)));
    else q.grid = std::max<int64_t>(1, std::min<int64_t>(p->grid * p->gpw / q.gpw, ceil_div(T, q.gpw)));
    *p = q;     // for the backward, the caller checks the workspace against the new grid
}

void log_policy(const char* op, int64_t T, int64_t H, const Policy& p)
{
    std::call_once(g_ovr_once, read_overrides);
    if (g_log)
        std::fprintf(stderr, "[rmsnorm_gfx950] %s T=%lld H=%lld lpr=%d nv=%d wgs=%d gpw=%d grid=%lld\n", op,
                     (long long)T, (long long)H, p.lpr, p.nv, p.wgs, p.gpw, (long long)p.grid);
}

// ---------------------------------------------------------------------------
// Validation helpers.
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Extent {
    uintptr_t lo, hi;   // [lo, hi)
};

Extent mat_extent(const void* p, int64_t T, int64_t H, int64_t ld, int64_t esize)
{
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + (uintptr_t)(((T - 1) * ld + H) * esize)};
}

Extent vec_extent(const void* p, int64_t n, int64_t esize)
{
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + (uintptr_t)(n * esize)};
}

bool overlap(const Extent& a, const Extent& b) { return a.lo < b.hi && b.lo < a.hi; }

bool valid_pair(int x_dtype, int w_dtype)
{
    return (x_dtype == RN_F32 && w_dtype == RN_F32) || (x_dtype == RN_BF16 && w_dtype == RN_BF16) ||
           (x_dtype == RN_BF16 && w_dtype == RN_F32);
}

int check_matrix(const void* p, int64_t ld, int64_t H, int dt)
{
    if (!aligned(p, 16)) return RN_ERR_ALIGN;
    if (ld < H || (ld * elem_bytes(dt)) % 16 != 0) return RN_ERR_STRIDE;
    return RN_OK;
}

int check_h(int64_t H, int dt)
{
    if (H <= 0 || H > RN_MAX_H) return RN_ERR_SHAPE;
    if (H % elems_per_chunk(dt) != 0) return RN_ERR_SHAPE;
    return RN_OK;
}

// Workspace bytes for G row strips: fp32 partials in blocks of 16 columns.
size_t workspace_need(int64_t G, int64_t H)
{
    const int64_t cols = (H + rn::RN_PART_COLS - 1) / rn::RN_PART_COLS * rn::RN_PART_COLS;
    return (size_t)G * (size_t)cols * sizeof(float);
}

// Clear a stale error left by earlier HIP calls on this thread, so that the
// error read after our launch is our own.
void clear_last_error() { (void)hipGetLastError(); }

// Same buffer, same row stride: an element-wise in-place update.
bool same_matrix(const void* a, int64_t lda, const void* b, int64_t ldb) { return a == b && lda == ldb; }

// Forward, plain or with a residual stream (u, h_out).
int fwd_common(const void* x, int64_t ldx, const void* u, int64_t ldu, int x_dtype, const void* w, int w_dtype,
               void* y, int64_t ldy, void* h, int64_t ldh, float* rstd, int64_t T, int64_t H, float eps,
               void* stream, bool residual)
{
    if (!valid_pair(x_dtype, w_dtype)) return RN_ERR_DTYPE;
    int st;
    if ((st = check_h(H, x_dtype)) != RN_OK) return st;
    if (T < 0) return RN_ERR_SHAPE;
    Policy p{};
    auto policy = [&](int cu, Policy* q) {
        return residual ? policy_fwd_residual(T, H, x_dtype, cu, q) : policy_fwd(T, H, x_dtype, cu, q);
    };
    if ((st = policy(1, &p)) != RN_OK) return st;                           // shape range (CU-independent)
    if (T == 0) return RN_OK;
    if (!x || !w || !y || !rstd) return RN_ERR_NULL;
    if (residual && (!u || !h)) return RN_ERR_NULL;
    if ((st = check_matrix(x, ldx, H, x_dtype)) != RN_OK) return st;
    if ((st = check_matrix(y, ldy, H, x_dtype)) != RN_OK) return st;
    if (residual) {
        if ((st = check_matrix(u, ldu, H, x_dtype)) != RN_OK) return st;
        if ((st = check_matrix(h, ldh, H, x_dtype)) != RN_OK) return st;
    }
    if (!aligned(w, 16) || !aligned(rstd, 4)) return RN_ERR_ALIGN;
    const int xb = elem_bytes(x_dtype);
    const Extent ex = mat_extent(x, T, H, ldx, xb), ey = mat_extent(y, T, H, ldy, xb);
    const Extent ew = vec_extent(w, H, elem_bytes(w_dtype)), er = vec_extent(rstd, T, 4);
    if (overlap(ey, ex) || overlap(ey, ew) || overlap(ey, er) || overlap(er, ex) || overlap(er, ew))
        return RN_ERR_ALIAS;
    if (residual) {
        const Extent eu = mat_extent(u, T, H, ldu, xb), eh = mat_extent(h, T, H, ldh, xb);
        if (overlap(ey, eu) || overlap(er, eu) || overlap(eh, ey) || overlap(eh, ew) || overlap(eh, er))
            return RN_ERR_ALIAS;
        if (overlap(eh, ex) && !same_matrix(h, ldh, x, ldx)) return RN_ERR_ALIAS;
        if (overlap(eh, eu) && !same_matrix(h, ldh, u, ldu)) return RN_ERR_ALIAS;
    }

    int cu = 0;
    if ((st = current_device_cu(&cu)) != RN_OK) return st;
    if ((st = policy(cu, &p)) != RN_OK) return st;
    apply_override(0, T, (int)(H / elems_per_chunk(x_dtype)), &p);
    log_policy(residual ? "fwd_residual" : "fwd", T, H, p);

    rn::FwdArgs a{};
    a.lpr = p.lpr;
    a.interleave = (p.flags & rn::RN_FLAG_ILV) ? 1 : 0;
    a.heads = 1;
    a.x = x; a.ldx = ldx;
    a.u = u; a.ldu = ldu;
    a.h = h; a.ldh = ldh;
    a.w = w;
    a.y = y; a.ldy = ldy;
    a.rstd = rstd;
    a.T = T; a.H = (int)H; a.nch = (int)(H / elems_per_chunk(x_dtype)); a.eps = eps;
    clear_last_error();
    if (rn::launch_fwd(a, x_dtype, w_dtype, residual ? rn::FWD_RESIDUAL : rn::FWD_PLAIN, p, (hipStream_t)stream) !=
        hipSuccess)
        return RN_ERR_LAUNCH;
    return RN_OK;
}

// The fused producer, every variant.
// need_normed: normed_out is required (the block-quant entry point).
int fp8_common(const void* x, int64_t ldx, void* residual, int64_t ldr, const void* w, int dtype, uint8_t* out,
               int64_t ldo, int fmt, float* block_scale, int64_t scale_ld, const float* tensor_scale,
               void* normed_out, int64_t ldn, int64_t T, int64_t H, float eps, void* stream, bool need_normed)
{
    if (dtype != RN_BF16 && dtype != RN_F16) return RN_ERR_DTYPE;
    if (fmt != RN_E4M3 && fmt != RN_E5M2) return RN_ERR_DTYPE;
    if (H <= 0 || H > RN_MAX_H || H % 128 != 0) return RN_ERR_SHAPE;
    if (T < 0) return RN_ERR_SHAPE;
    int st;
    Policy p{};
    if ((st = policy_fp8(T, H, 1, &p)) != RN_OK) return st;               // shape range (CU-independent)
    if (T == 0) return RN_OK;
    if (!x || !residual || !w || !out || (need_normed && !normed_out)) return RN_ERR_NULL;
    const bool tsc = tensor_scale != nullptr;
    if (tsc == (block_scale != nullptr)) return RN_ERR_NULL;              // exactly one scale form
    if ((st = check_matrix(x, ldx, H, RN_BF16)) != RN_OK) return st;      // 16-bit rows either way
    if ((st = check_matrix(residual, ldr, H, RN_BF16)) != RN_OK) return st;
    if (normed_out && (st = check_matrix(normed_out, ldn, H, RN_BF16)) != RN_OK) return st;
    if (!aligned(out, 16)) return RN_ERR_ALIGN;
    if (ldo < H || ldo % 16 != 0) return RN_ERR_STRIDE;
    if (!aligned(w, 16)) return RN_ERR_ALIGN;
    if (tsc ? !aligned(tensor_scale, 4) : !aligned(block_scale, 4)) return RN_ERR_ALIGN;
    if (!tsc && (scale_ld < T || scale_ld % 4 != 0)) return RN_ERR_STRIDE;
    const Extent ex = mat_extent(x, T, H, ldx, 2), er = mat_extent(residual, T, H, ldr, 2);
    const Extent ew = vec_extent(w, H, 2), eo = mat_extent(out, T, H, ldo, 1);
    const Extent en = normed_out ? mat_extent(normed_out, T, H, ldn, 2) : Extent{0, 0};
    const Extent es = tsc ? vec_extent(tensor_scale, 1, 4)
                          : Extent{reinterpret_cast<uintptr_t>(block_scale),
                                   reinterpret_cast<uintptr_t>(block_scale) + (uintptr_t)(((H / 128 - 1) * scale_ld + T) * 4)};
    // Outputs: residual (in place), out, normed, and the block scales.  The
    // per-tensor scale is an input: only the outputs may not overlap it.
    if (overlap(er, ex) || overlap(er, ew) || overlap(eo, ex) || overlap(eo, er) || overlap(eo, ew) ||
        overlap(eo, en) || overlap(eo, es) || overlap(en, ex) || overlap(en, er) || overlap(en, ew) ||
        overlap(en, es) || overlap(es, er) || (!tsc && (overlap(es, ex) || overlap(es, ew))))
        return RN_ERR_ALIAS;

    int cu = 0;
    if ((st = current_device_cu(&cu)) != RN_OK) return st;
    if ((st = policy_fp8(T, H, cu, &p)) != RN_OK) return st;
    apply_override(2, T, (int)(H / 8), &p);
    log_policy("fp8", T, H, p);

    rn::Fp8Args a{};
    a.lpr = p.lpr;
    a.interleave = (p.flags & rn::RN_FLAG_ILV) ? 1 : 0;
    a.x = x; a.ldx = ldx;
    a.res = residual; a.ldr = ldr;
    a.w = w;
    a.out = out; a.ldo = ldo;
    a.scale = block_scale; a.scale_ld = scale_ld;
    a.tscale = tensor_scale;
    a.normed = normed_out; a.ldn = ldn;
    a.T = T; a.H = (int)H; a.nch = (int)(H / 8); a.eps = eps;
    clear_last_error();
    if (rn::launch_fp8(a, dtype, fmt, tsc, p, (hipStream_t)stream) != hipSuccess)
        return RN_ERR_LAUNCH;
    return RN_OK;
}

// Extent of a per-head tensor: T tokens of `heads` rows of D elements.
Extent heads_extent(const void* p, int64_t T, int64_t heads, int64_t D, int64_t ld_t, int64_t ld_h, int64_t esize)
{
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + (uintptr_t)(((T - 1) * ld_t + (heads - 1) * ld_h + D) * esize)};
}

// Strides of a per-head tensor: heads of one token do not overlap and lie
// inside the token's stride; both strides are 16-byte multiples.
int check_heads(const void* p, int64_t ld_t, int64_t ld_h, int64_t heads, int64_t D, int dt)
{
    if (!aligned(p, 16)) return RN_ERR_ALIGN;
    const int64_t es = elem_bytes(dt);
    if ((ld_h * es) % 16 != 0 || (ld_t * es) % 16 != 0) return RN_ERR_STRIDE;
    if (heads > 1 && ld_h < D) return RN_ERR_STRIDE;
    if (ld_t < (heads - 1) * ld_h + D) return RN_ERR_STRIDE;
    return RN_OK;
}

// Backward, plain or with the residual-stream gradient g_residual.
int bwd_common(const void* dy, int64_t lddy, const void* x, int64_t ldx, int x_dtype, const void* w, int w_dtype,
               const float* rstd, const void* gres, int64_t ldgr, void* dx, int64_t lddx, float* dw, int64_t T,
               int64_t H, int deterministic, void* workspace, size_t workspace_bytes, void* stream, bool residual,
               bool use_scratch = false)
{
    if (!valid_pair(x_dtype, w_dtype)) return RN_ERR_DTYPE;
    int st;
    if ((st = check_h(H, x_dtype)) != RN_OK) return st;
    if (T < 0) return RN_ERR_SHAPE;
    Policy p{};
    if ((st = policy_bwd(T, H, x_dtype, 1, &p)) != RN_OK) return st;      // shape range (CU-independent)
    if (!dw) return RN_ERR_NULL;
    if (!aligned(dw, 4)) return RN_ERR_ALIGN;
    const int xb = elem_bytes(x_dtype);
    const Extent edw = vec_extent(dw, H, 4);
    Extent edy{}, ex{}, edx{}, ew{}, er{}, eg{};
    if (T > 0) {
        if (!dy || !x || !w || !rstd || !dx) return RN_ERR_NULL;
        if (residual && !gres) return RN_ERR_NULL;
        if ((st = check_matrix(dy, lddy, H, x_dtype)) != RN_OK) return st;
        if ((st = check_matrix(x, ldx, H, x_dtype)) != RN_OK) return st;
        if ((st = check_matrix(dx, lddx, H, x_dtype)) != RN_OK) return st;
        if (residual && (st = check_matrix(gres, ldgr, H, x_dtype)) != RN_OK) return st;
        if (!aligned(w, 16) || !aligned(rstd, 4)) return RN_ERR_ALIGN;
        edy = mat_extent(dy, T, H, lddy, xb);
        ex = mat_extent(x, T, H, ldx, xb);
        edx = mat_extent(dx, T, H, lddx, xb);
        ew = vec_extent(w, H, elem_bytes(w_dtype));
        er = vec_extent(rstd, T, 4);
        if (overlap(edx, edy) || overlap(edx, ex) || overlap(edx, ew) || overlap(edx, er) || overlap(edx, edw) ||
            overlap(edw, edy) || overlap(edw, ex) || overlap(edw, ew) || overlap(edw, er))
            return RN_ERR_ALIAS;
        if (residual) {
            eg = mat_extent(gres, T, H, ldgr, xb);
            if (overlap(edw, eg)) return RN_ERR_ALIAS;
            if (overlap(edx, eg) && !same_matrix(dx, lddx, gres, ldgr)) return RN_ERR_ALIAS;
        }
        // Only a launch of several row strips keeps partial sums in the workspace.
        if (!use_scratch && !bwd_one_strip(T, H, x_dtype)) {
            if (!workspace) return RN_ERR_WORKSPACE;
            if (!aligned(workspace, 16)) return RN_ERR_ALIGN;
        }
    }

    int cu = 0;
    if ((st = current_device_cu(&cu)) != RN_OK) return st;
    clear_last_error();
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        // No rows: the weight gradient is the empty sum.
        if (rn::launch_fill_zero(dw, H, s) != hipSuccess) return RN_ERR_LAUNCH;
        return RN_OK;
    }
    if ((st = residual ? policy_bwd_residual(T, H, x_dtype, cu, &p) : policy_bwd(T, H, x_dtype, cu, &p)) != RN_OK)
        return st;
    apply_override(1, T, (int)(H / elems_per_chunk(x_dtype)), &p);
    log_policy(residual ? "bwd_residual" : "bwd", T, H, p);
    // With one row strip its partial is the column sum itself: it goes
    // straight into dw, with no second launch and no workspace (the same bits
    // as the reduce of a single partial, which only widens it to FP64 and
    // back).  A device with a single CU gets one strip for any T; the
    // workspace was required above all the same.
    const bool direct = p.grid == 1;
    if (!direct && use_scratch) {
        float* sp = nullptr;
        if (workspace_need(p.grid, H) > kScratchFloats * sizeof(float)) return RN_ERR_WORKSPACE;
        if ((st = current_scratch(&sp)) != RN_OK) return st;
        clear_last_error();
        workspace = sp;
        workspace_bytes = kScratchFloats * sizeof(float);
    }
    if (!direct) {
        const size_t need = workspace_need(p.grid, H);
        if (!workspace) return RN_ERR_WORKSPACE;
        if (workspace_bytes < need) return RN_ERR_WORKSPACE;
        const Extent ews = vec_extent(workspace, (int64_t)(need / 4), 4);
        if (overlap(ews, edy) || overlap(ews, ex) || overlap(ews, ew) || overlap(ews, er) || overlap(ews, edx) ||
            overlap(ews, edw) || (residual && overlap(ews, eg)))
            return RN_ERR_ALIAS;
    }

    rn::BwdArgs a{};
    a.lpr = p.lpr;
    a.interleave = (p.flags & rn::RN_FLAG_ILV) ? 1 : 0;
    a.dy = dy; a.lddy = lddy;
    a.x = x; a.ldx = ldx;
    a.w = w;
    a.rstd = rstd;
    a.gres = gres; a.ldgr = ldgr;
    a.dx = dx; a.lddx = lddx;
    a.T = T; a.H = (int)H; a.nch = (int)(H / elems_per_chunk(x_dtype));
    a.inv_h = 1.0f / (float)H;
    // Both values of the flag run the same fixed-order reduction and give the
    // same bits (see the header).
    (void)deterministic;
    a.part = direct ? dw : static_cast<float*>(workspace);
    a.part_vec = aligned(a.part, 16) ? 1 : 0;
    if (rn::launch_bwd(a, x_dtype, w_dtype, residual ? 1 : 0, p, s) != hipSuccess) return RN_ERR_LAUNCH;
    if (!direct) {
        rn::ReduceArgs ra{static_cast<const float*>(workspace), dw, p.grid, (int)H};
        if (rn::launch_bwd_reduce(ra, s) != hipSuccess) return RN_ERR_LAUNCH;
    }
    return RN_OK;
}

} // namespace

// ===========================================================================
// Exported C ABI.
// ===========================================================================
extern "C" {

const char* rn_status_string(int status)
{
    switch (status) {
    case RN_OK: return "ok";
    case RN_ERR_NULL: return "null pointer";
    case RN_ERR_SHAPE: return "unsupported shape";
    case RN_ERR_DTYPE: return "unsupported dtype";
    case RN_ERR_ALIGN: return "misaligned pointer";
    case RN_ERR_STRIDE: return "bad row stride";
    case RN_ERR_WORKSPACE: return "workspace missing or too small";
    case RN_ERR_ALIAS: return "overlapping buffers";
    case RN_ERR_DEVICE: return "no gfx950 device";
    case RN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int rn_version(void) { return 10000; }

int rn_query_policy(int op, int64_t T, int64_t H, int x_dtype, int w_dtype, int cu_count, int32_t* out)
{
    if (!out) return RN_ERR_NULL;
    if (cu_count <= 0 || T < 0) return RN_ERR_SHAPE;
    Policy p{};
    int st;
    if (op == 0 || op == 1 || op == 3 || op == 4) {
        if (!valid_pair(x_dtype, w_dtype)) return RN_ERR_DTYPE;
        if ((st = check_h(H, x_dtype)) != RN_OK) return st;
        st = op == 1 ? policy_bwd(T, H, x_dtype, cu_count, &p)
           : op == 3 ? policy_fwd_residual(T, H, x_dtype, cu_count, &p)
           : op == 4 ? policy_bwd_residual(T, H, x_dtype, cu_count, &p)
                     : policy_fwd(T, H, x_dtype, cu_count, &p);
    } else if (op == 2) {
        if (x_dtype != RN_BF16 || w_dtype != RN_BF16) return RN_ERR_DTYPE;
        if (H <= 0 || H > RN_MAX_H || H % 128 != 0) return RN_ERR_SHAPE;
        st = policy_fp8(T, H, cu_count, &p);
    } else {
        return RN_ERR_SHAPE;
    }
    if (st != RN_OK) return st;
    out[0] = p.lpr; out[1] = p.nv; out[2] = p.wgs; out[3] = (int32_t)p.grid; out[4] = p.gpw; out[5] = p.kernel;
    out[6] = p.flags;
    return RN_OK;
}

size_t rn_bwd_workspace_bytes_for(int64_t T, int64_t H, int cu_count)
{
    if (T < 0 || H <= 0 || H > RN_MAX_H || cu_count <= 0) return (size_t)-1;
    if (T == 0) return 0;
    Policy p{};
    // The bf16 and f32 policies give the same strip count bound (<= cu_count);
    // size for the larger of the two so one workspace serves both.  A launch
    // of one strip needs none.
    size_t best = 0;
    bool any = false;
    for (int dt = 0; dt < 2; ++dt) {
        if (H % elems_per_chunk(dt) != 0) continue;
        if (policy_bwd(T, H, dt, cu_count, &p) != RN_OK) continue;
        any = true;
        if (bwd_one_strip(T, H, dt)) continue;
        const size_t b = workspace_need(p.grid, H);
        if (b > best) best = b;
    }
    if (!any) return (size_t)-1;
    return (best + 255) / 256 * 256;
}

size_t rmsnorm_bwd_workspace_bytes(int64_t T, int64_t H, int device)
{
    int cu = 0;
    if (device_cu(device, &cu) != RN_OK) return (size_t)-1;
    return rn_bwd_workspace_bytes_for(T, H, cu);
}

int rmsnorm_fwd(const void* x, int64_t ldx, int x_dtype, const void* w, int w_dtype, void* y, int64_t ldy,
                float* rstd, int64_t T, int64_t H, float eps, void* stream)
{
    return fwd_common(x, ldx, nullptr, 0, x_dtype, w, w_dtype, y, ldy, nullptr, 0, rstd, T, H, eps, stream, false);
}

int rmsnorm_fwd_residual(const void* x, int64_t ldx, const void* u, int64_t ldu, int x_dtype, const void* w,
                         int w_dtype, void* y, int64_t ldy, void* h_out, int64_t ldh, float* rstd, int64_t T,
                         int64_t H, float eps, void* stream)
{
    return fwd_common(x, ldx, u, ldu, x_dtype, w, w_dtype, y, ldy, h_out, ldh, rstd, T, H, eps, stream, true);
}

int rmsnorm_fwd_heads(const void* x, int64_t ld_token, int64_t ld_head, int x_dtype, const void* w, int w_dtype,
                      void* y, int64_t ldy_token, int64_t ldy_head, float* rstd, int64_t T, int64_t heads,
                      int64_t head_dim, float eps, void* stream)
{
    if (!valid_pair(x_dtype, w_dtype)) return RN_ERR_DTYPE;
    const int64_t D = head_dim;
    int st;
    if ((st = check_h(D, x_dtype)) != RN_OK) return st;
    if (D / elems_per_chunk(x_dtype) > RN_HEADS_MAX_VECTORS) return RN_ERR_SHAPE;
    if (T < 0 || heads < 1 || heads > 65535) return RN_ERR_SHAPE;
    if (T * heads > (int64_t)INT32_MAX) return RN_ERR_SHAPE;
    const int64_t rows = T * heads;
    Policy p{};
    if ((st = policy_fwd(rows, D, x_dtype, 1, &p)) != RN_OK) return st;
    if (rows == 0) return RN_OK;
    if (!x || !w || !y) return RN_ERR_NULL;
    if ((st = check_heads(x, ld_token, ld_head, heads, D, x_dtype)) != RN_OK) return st;
    if ((st = check_heads(y, ldy_token, ldy_head, heads, D, x_dtype)) != RN_OK) return st;
    if (!aligned(w, 16) || (rstd && !aligned(rstd, 4))) return RN_ERR_ALIGN;
    const int xb = elem_bytes(x_dtype);
    const Extent ex = heads_extent(x, T, heads, D, ld_token, ld_head, xb);
    const Extent ey = heads_extent(y, T, heads, D, ldy_token, ldy_head, xb);
    const Extent ew = vec_extent(w, D, elem_bytes(w_dtype));
    const bool in_place = x == y && ld_token == ldy_token && (heads == 1 || ld_head == ldy_head);
    if (overlap(ey, ex) && !in_place) return RN_ERR_ALIAS;
    if (overlap(ey, ew)) return RN_ERR_ALIAS;
    if (rstd) {
        const Extent er = vec_extent(rstd, rows, 4);
        if (overlap(er, ex) || overlap(er, ey) || overlap(er, ew)) return RN_ERR_ALIAS;
    }

    int cu = 0;
    if ((st = current_device_cu(&cu)) != RN_OK) return st;
    if ((st = policy_fwd(rows, D, x_dtype, cu, &p)) != RN_OK) return st;
    apply_override(0, rows, (int)(D / elems_per_chunk(x_dtype)), &p);
    if (p.lpr >= 64) return RN_ERR_SHAPE;                 // only sub-wave row groups serve this form
    log_policy("fwd_heads", rows, D, p);

    rn::FwdArgs a{};
    a.lpr = p.lpr;
    a.interleave = (p.flags & rn::RN_FLAG_ILV) ? 1 : 0;
    a.heads = (int)heads;
    {
        // floor(r / heads) = (r * m) >> (31 + l) for r < 2^31: l = ceil(log2 heads),
        // m = ceil(2^(31+l) / heads), which is below 2^32.
        int l = 0;
        while ((int64_t(1) << l) < heads) ++l;
        const uint64_t m = ((uint64_t(1) << (31 + l)) + (uint64_t)heads - 1) / (uint64_t)heads;
        a.hmul = (uint32_t)m;
        a.hshift = 31 + l;
    }
    a.x = x; a.ldx = ld_token; a.ldxh = ld_head;
    a.w = w;
    a.y = y; a.ldy = ldy_token; a.ldyh = ldy_head;
    a.rstd = rstd;
    a.T = rows; a.H = (int)D; a.nch = (int)(D / elems_per_chunk(x_dtype)); a.eps = eps;
    clear_last_error();
    if (rn::launch_fwd(a, x_dtype, w_dtype, rn::FWD_HEADS, p, (hipStream_t)stream) != hipSuccess) return RN_ERR_LAUNCH;
    return RN_OK;
}

int rmsnorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, int x_dtype, const void* w, int w_dtype,
                const float* rstd, void* dx, int64_t lddx, float* dw, int64_t T, int64_t H, int deterministic,
                void* workspace, size_t workspace_bytes, void* stream)
{
    return bwd_common(dy, lddy, x, ldx, x_dtype, w, w_dtype, rstd, nullptr, 0, dx, lddx, dw, T, H, deterministic,
                      workspace, workspace_bytes, stream, false);
}

int rmsnorm_bwd_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx, int x_dtype, const void* w,
                        int w_dtype, const float* rstd, void* dx, int64_t lddx, float* dw, int64_t T, int64_t H,
                        int deterministic, void* stream)
{
    return bwd_common(dy, lddy, x, ldx, x_dtype, w, w_dtype, rstd, nullptr, 0, dx, lddx, dw, T, H, deterministic,
                      nullptr, 0, stream, false, true);
}

int rmsnorm_bwd_residual(const void* dy, int64_t lddy, const void* x, int64_t ldx, int x_dtype, const void* w,
                         int w_dtype, const float* rstd, const void* g_residual, int64_t ldgr, void* dx,
                         int64_t lddx, float* dw, int64_t T, int64_t H, int deterministic, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    return bwd_common(dy, lddy, x, ldx, x_dtype, w, w_dtype, rstd, g_residual, ldgr, dx, lddx, dw, T, H,
                      deterministic, workspace, workspace_bytes, stream, true);
}

int add_rmsnorm_fp8_block_quant(const void* x, int64_t ldx, void* residual, int64_t ldr, const void* w,
                                uint8_t* out, int64_t ldo, float* block_scale, int64_t scale_ld, void* normed_out,
                                int64_t ldn, int64_t T, int64_t H, float eps, void* stream)
{
    return fp8_common(x, ldx, residual, ldr, w, RN_BF16, out, ldo, RN_E4M3, block_scale, scale_ld, nullptr,
                      normed_out, ldn, T, H, eps, stream, true);
}

int add_rmsnorm_fp8_quant(const void* x, int64_t ldx, void* residual, int64_t ldr, const void* w, int dtype,
                          uint8_t* out, int64_t ldo, int out_format, float* block_scale, int64_t scale_ld,
                          const float* tensor_scale, void* normed_out, int64_t ldn, int64_t T, int64_t H,
                          float eps, void* stream)
{
    return fp8_common(x, ldx, residual, ldr, w, dtype, out, ldo, out_format, block_scale, scale_ld, tensor_scale,
                      normed_out, ldn, T, H, eps, stream, false);
}

} // extern "C"

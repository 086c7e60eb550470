// attend.hip -- dispatch of the split kernel, occupancy queries, the
// fixed-order merge of the per-split partials, and the fill of an empty
// segment's result.
#include <atomic>

#include "common.h"

namespace rkv {

#define RKV_DECL(kt, vt)                                                                                  \
    hipError_t launch_split_k##kt##_v##vt(int d, int rt, dim3 grid, const float *q, float *pa, float2 *pm, \
                                          float *o, float *lse, const SplitParams &p, hipStream_t s);       \
    int split_waves_k##kt##_v##vt(int d, int rt);                                                         \
    int split_occupancy_k##kt##_v##vt(int d, int rt);                                                     \
    hipError_t launch_split_shd_k##kt##_v##vt(dim3 grid, const float *q, float *pa, float2 *pm, float *o, \
                                              float *lse, const SplitParams &p, hipStream_t s);           \
    int split_shd_occupancy_k##kt##_v##vt();                                                              \
    bool split_shd_supported_k##kt##_v##vt();
#define RKV_DECL_K(kt) RKV_DECL(kt, 0) RKV_DECL(kt, 1) RKV_DECL(kt, 2) RKV_DECL(kt, 3) RKV_DECL(kt, 4)
RKV_DECL_K(0)
RKV_DECL_K(1)
RKV_DECL_K(2)
RKV_DECL_K(3)

bool split_supported(int kt, int vt, int d, int rt)
{
    const bool t = kt >= 0 && kt <= 3 && vt >= 0 && vt <= 4;
    const bool dd = (d == 64 && vt != kT3) || d == 128 || d == 256 || (d == 512 && kt != kF32 && vt != kF32);
    const bool r = rt == 1 || rt == 2 || rt == 4 || rt == 5 || rt == 8 || rt == 16;
    return t && dd && r;
}

int split_dim_slices(int kt, int vt, int d)
{
    const bool blk = (kt == kQ8 || kt == kQ4) && (vt == kQ8 || vt == kQ4 || vt == kT3);
    return blk && d > 128 ? d / 128 : 1;
}

int split_waves(int kt, int vt, int d, int rt)
{
#define RKV_NW(kk, vv) \
    if (kt == kk && vt == vv) return split_waves_k##kk##_v##vv(d, rt);
#define RKV_NW_K(kk) RKV_NW(kk, 0) RKV_NW(kk, 1) RKV_NW(kk, 2) RKV_NW(kk, 3) RKV_NW(kk, 4)
    RKV_NW_K(0)
    RKV_NW_K(1)
    RKV_NW_K(2)
    RKV_NW_K(3)
    return 0;
}

int split_occupancy(int kt, int vt, int d, int rt)
{
    // cached per instance and device (the first query on a device may be
    // slow); atomics, since calls may plan from several host threads
    static std::atomic<int> cache[4][5][4][6][16];
    static const int rts[6] = {1, 2, 4, 5, 8, 16};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    int ri = -1;
    for (int i = 0; i < 6; ++i)
        if (rts[i] == rt) ri = i;
    const int di = d == 64 ? 0 : d == 128 ? 1 : d == 256 ? 2 : d == 512 ? 3 : -1;
    if (ri < 0 || di < 0 || kt < 0 || kt > 3 || vt < 0 || vt > 4 || dev < 0 || dev >= 16) return 0;
    std::atomic<int> &slot = cache[kt][vt][di][ri][dev];
    int c = slot.load(std::memory_order_relaxed);
    if (c == 0) {
#define RKV_OCC(kk, vv) \
    if (kt == kk && vt == vv) c = split_occupancy_k##kk##_v##vv(d, rt);
#define RKV_OCC_K(kk) RKV_OCC(kk, 0) RKV_OCC(kk, 1) RKV_OCC(kk, 2) RKV_OCC(kk, 3) RKV_OCC(kk, 4)
        RKV_OCC_K(0)
        RKV_OCC_K(1)
        RKV_OCC_K(2)
        RKV_OCC_K(3)
        if (c <= 0) c = -1;
        slot.store(c, std::memory_order_relaxed);  // every thread computes the same value
    }
    return c > 0 ? c : 0;
}

int compute_units()
{
    static std::atomic<int> cu[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 0;
    }
    int n = cu[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = -1;
        }
        cu[dev].store(n, std::memory_order_relaxed);
    }
    return n > 0 ? n : 0;
}

bool split_shd_supported(int kt, int vt)
{
#define RKV_SOK(kk, vv) \
    if (kt == kk && vt == vv) return split_shd_supported_k##kk##_v##vv();
#define RKV_SOK_K(kk) RKV_SOK(kk, 0) RKV_SOK(kk, 1) RKV_SOK(kk, 2) RKV_SOK(kk, 3) RKV_SOK(kk, 4)
    RKV_SOK_K(0)
    RKV_SOK_K(1)
    RKV_SOK_K(2)
    RKV_SOK_K(3)
    return false;
}

int split_shd_occupancy(int kt, int vt)
{
    static std::atomic<int> cache[4][5][16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (kt < 0 || kt > 3 || vt < 0 || vt > 4 || dev < 0 || dev >= 16) return 0;
    std::atomic<int> &slot = cache[kt][vt][dev];
    int c = slot.load(std::memory_order_relaxed);
    if (c == 0) {
#define RKV_SOCC(kk, vv) \
    if (kt == kk && vt == vv) c = split_shd_occupancy_k##kk##_v##vv();
#define RKV_SOCC_K(kk) RKV_SOCC(kk, 0) RKV_SOCC(kk, 1) RKV_SOCC(kk, 2) RKV_SOCC(kk, 3) RKV_SOCC(kk, 4)
        RKV_SOCC_K(0)
        RKV_SOCC_K(1)
        RKV_SOCC_K(2)
        RKV_SOCC_K(3)
        if (c <= 0) c = -1;
        slot.store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

hipError_t launch_split_shd(int kt, int vt, dim3 grid, const float *q, float *pa, float2 *pm, float *o, float *lse,
                            const SplitParams &p, hipStream_t s)
{
#define RKV_SCASE(kk, vv) \
    if (kt == kk && vt == vv) return launch_split_shd_k##kk##_v##vv(grid, q, pa, pm, o, lse, p, s);
#define RKV_SCASE_K(kk) RKV_SCASE(kk, 0) RKV_SCASE(kk, 1) RKV_SCASE(kk, 2) RKV_SCASE(kk, 3) RKV_SCASE(kk, 4)
    RKV_SCASE_K(0)
    RKV_SCASE_K(1)
    RKV_SCASE_K(2)
    RKV_SCASE_K(3)
    return hipErrorInvalidValue;
}

hipError_t launch_split(int kt, int vt, int d, int rt, dim3 grid, const float *q, float *pa, float2 *pm, float *o,
                        float *lse, const SplitParams &p, hipStream_t s)
{
#define RKV_CASE(kk, vv) \
    if (kt == kk && vt == vv) return launch_split_k##kk##_v##vv(d, rt, grid, q, pa, pm, o, lse, p, s);
#define RKV_CASE_K(kk) RKV_CASE(kk, 0) RKV_CASE(kk, 1) RKV_CASE(kk, 2) RKV_CASE(kk, 3) RKV_CASE(kk, 4)
    RKV_CASE_K(0)
    RKV_CASE_K(1)
    RKV_CASE_K(2)
    RKV_CASE_K(3)
    return hipErrorInvalidValue;
}

// Merge of the per-split partials of one row (partials are in log2 units):
// M = max_i m_i, L = sum_i l_i 2^(m_i - M), o = sum_i acc_i 2^(m_i - M) / L,
// lse = (M + log2 L) ln 2.  Block (row, 32-dim slice) of 256 threads: 32
// groups of 8 lanes, lane c holding 4 dims; group j takes splits j, j+32,
// j+64, ...  The row's maximum M is found first (thread t reads the (m, l) of
// splits t, t+256, ..., a block reduction), so every weight 2^(m_i - M) is
// independent of the others (no running rescale); the weighted sums are added
// per group in split order and then over the groups in group order: the
// result does not depend on timing.  The loads of the weighted pass are
// issued before the maximum is known.  If `done` is given, one thread writes
// done_value there (host-visible memory, system scope) as the kernel starts:
// the split kernel before it has then finished reading its key tiles.
// o_x / lse_x (optional): a normalised part (O and natural-log LSE, i.e. the
// partial acc = O, m = LSE log2 e, l = 1), merged first; lse = -inf gives it
// weight 0.
__device__ __forceinline__ float block_max256(float v, float *sw)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int t = threadIdx.x;
    if ((t & 63) == 0) sw[t >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(sw[0], sw[1]), fmaxf(sw[2], sw[3]));
}

__global__ void __launch_bounds__(256)
rkv_reduce_kernel(const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int n_splits,
                  int64_t n_rows, int D, float *__restrict__ o, float *__restrict__ lse, uint64_t *done,
                  uint64_t done_value, const float *__restrict__ o_x, const float *__restrict__ lse_x)
{
    if (done && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        __hip_atomic_store(done, done_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __shared__ float sW[4], sL[32];
    __shared__ float4 sA[32][8];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, grp = t >> 3, c = t & 7;
    const int d0 = blockIdx.y * 32 + 4 * c;
    const float2 *ml_row = part_ml + row * n_splits;  // (m, l) are row-major: a row's splits are contiguous
    auto load = [&](int base, float2 (&ml)[8], float4 (&x)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // (indices past the end are neither loaded nor added)
            const int sp = base + 32 * u;
            if (sp < n_splits) {
                ml[u] = ml_row[sp];
                x[u] = *(const float4 *)(part_acc + ((int64_t)sp * n_rows + row) * D + d0);
            } else {
                ml[u] = make_float2(-INFINITY, 0.f);
                x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    float2 ml[8];
    float4 x[8];
    if (grp < n_splits) load(grp, ml, x);
    float mloc = -INFINITY;
    for (int sp = t; sp < n_splits; sp += 256) mloc = fmaxf(mloc, ml_row[sp].x);
    const float mx = lse_x ? lse_x[row] * 1.4426950408889634f : -INFINITY;  // the extra part, log2 units
    const float M = fmaxf(block_max256(mloc, sW), mx);
    float l = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = grp; base < n_splits; base += 32 * 8) {
        if (base != grp) load(base, ml, x);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (base + 32 * u < n_splits) {
                const float w = ml[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - M);
                l = fmaf(ml[u].y, w, l);
                a.x = fmaf(x[u].x, w, a.x);
                a.y = fmaf(x[u].y, w, a.y);
                a.z = fmaf(x[u].z, w, a.z);
                a.w = fmaf(x[u].w, w, a.w);
            }
        }
    }
    if (c == 0) sL[grp] = l;
    sA[grp][c] = a;
    __syncthreads();
    if (grp == 0) {
        float L = 0.f;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (mx != -INFINITY) {
            const float w = __builtin_amdgcn_exp2f(mx - M);
            const float4 x = *(const float4 *)(o_x + row * D + d0);
            L = w;
            s = make_float4(x.x * w, x.y * w, x.z * w, x.w * w);
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            L += sL[j];
            s.x += sA[j][c].x;
            s.y += sA[j][c].y;
            s.z += sA[j][c].z;
            s.w += sA[j][c].w;
        }
        // a row that saw no key in any split: o = 0, lse = -inf
        *(float4 *)(o + row * D + d0) = L > 0.f ? make_float4(s.x / L, s.y / L, s.z / L, s.w / L)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
        if (blockIdx.y == 0 && c == 0) lse[row] = (M + log2f(L)) * 0.69314718055994531f;
    }
}

hipError_t launch_reduce(int d, int64_t n_rows, int n_splits, const float *pa, const float2 *pm, float *o,
                         float *lse, hipStream_t s, uint64_t *done, uint64_t done_value, const float *o_x,
                         const float *lse_x)
{
    if (d % 32 || n_rows <= 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)n_rows, (unsigned)(d / 32)), block(256);
    hipLaunchKernelGGL(rkv_reduce_kernel, grid, block, 0, s, pa, pm, n_splits, n_rows, d, o, lse, done, done_value,
                       o_x, lse_x);
    return hipGetLastError();
}

// The same signal on its own (when no merge follows the split kernel).
__global__ void __launch_bounds__(64) rkv_signal_kernel(uint64_t *done, uint64_t done_value)
{
    if (threadIdx.x == 0) __hip_atomic_store(done, done_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_signal(uint64_t *done, uint64_t done_value, hipStream_t s)
{
    hipLaunchKernelGGL(rkv_signal_kernel, dim3(1), dim3(64), 0, s, done, done_value);
    return hipGetLastError();
}

// Empty segment: o = 0, lse = -inf.
__global__ void __launch_bounds__(256) rkv_fill_empty_kernel(int d, int64_t n_rows, float *o, float *lse)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_rows * d) o[i] = 0.f;
    if (i < n_rows) lse[i] = -INFINITY;
}

hipError_t launch_fill_empty(int d, int64_t n_rows, float *o, float *lse, hipStream_t s)
{
    const int64_t n = n_rows * d;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rkv_fill_empty_kernel, dim3(blocks), dim3(256), 0, s, d, n_rows, o, lse);
    return hipGetLastError();
}

}  // namespace rkv

// attend.hip -- dispatch of the split kernel, occupancy queries, the
// fixed-order merge of the per-split partials, and the fill of an empty
// segment's result.
#include "common.h"

namespace rkv {

#define RKV_DECL(kt, vt)                                                                                  \
    hipError_t launch_split_k##kt##_v##vt(int d, int rt, dim3 grid, const float *q, float *pa, float2 *pm, \
                                          float *o, float *lse, const SplitParams &p, hipStream_t s);       \
    int split_waves_k##kt##_v##vt(int d);                                                                 \
    int split_occupancy_k##kt##_v##vt(int d, int rt);
#define RKV_DECL_K(kt) RKV_DECL(kt, 0) RKV_DECL(kt, 1) RKV_DECL(kt, 2) RKV_DECL(kt, 3)
RKV_DECL_K(0)
RKV_DECL_K(1)
RKV_DECL_K(2)
RKV_DECL_K(3)

bool split_supported(int kt, int vt, int d, int rt)
{
    const bool t = kt >= 0 && kt <= 3 && vt >= 0 && vt <= 3;
    const bool dd = d == 64 || d == 128 || d == 256 || (d == 512 && kt != kF32 && vt != kF32);
    const bool r = rt == 1 || rt == 2 || rt == 4 || rt == 5 || rt == 8 || rt == 16;
    return t && dd && r;
}

int split_waves(int kt, int vt, int d)
{
#define RKV_NW(kk, vv) \
    if (kt == kk && vt == vv) return split_waves_k##kk##_v##vv(d);
#define RKV_NW_K(kk) RKV_NW(kk, 0) RKV_NW(kk, 1) RKV_NW(kk, 2) RKV_NW(kk, 3)
    RKV_NW_K(0)
    RKV_NW_K(1)
    RKV_NW_K(2)
    RKV_NW_K(3)
    return 0;
}

int split_occupancy(int kt, int vt, int d, int rt)
{
    // cached per instance and device (the first query on a device may be slow)
    static int cache[4][4][4][6][16];
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
    if (ri < 0 || di < 0 || kt < 0 || kt > 3 || vt < 0 || vt > 3 || dev < 0 || dev >= 16) return 0;
    int &c = cache[kt][vt][di][ri][dev];
    if (c == 0) {
#define RKV_OCC(kk, vv) \
    if (kt == kk && vt == vv) c = split_occupancy_k##kk##_v##vv(d, rt);
#define RKV_OCC_K(kk) RKV_OCC(kk, 0) RKV_OCC(kk, 1) RKV_OCC(kk, 2) RKV_OCC(kk, 3)
        RKV_OCC_K(0)
        RKV_OCC_K(1)
        RKV_OCC_K(2)
        RKV_OCC_K(3)
        if (c <= 0) c = -1;
    }
    return c > 0 ? c : 0;
}

int compute_units()
{
    static int cu[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 0;
    }
    if (cu[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = -1;
        }
        cu[dev] = n;
    }
    return cu[dev] > 0 ? cu[dev] : 0;
}

hipError_t launch_split(int kt, int vt, int d, int rt, dim3 grid, const float *q, float *pa, float2 *pm, float *o,
                        float *lse, const SplitParams &p, hipStream_t s)
{
#define RKV_CASE(kk, vv) \
    if (kt == kk && vt == vv) return launch_split_k##kk##_v##vv(d, rt, grid, q, pa, pm, o, lse, p, s);
#define RKV_CASE_K(kk) RKV_CASE(kk, 0) RKV_CASE(kk, 1) RKV_CASE(kk, 2) RKV_CASE(kk, 3)
    RKV_CASE_K(0)
    RKV_CASE_K(1)
    RKV_CASE_K(2)
    RKV_CASE_K(3)
    return hipErrorInvalidValue;
}

// Merge of the per-range partials of one row (partials are in log2 units):
// M = max_i m_i, L = sum_i l_i 2^(m_i - M), o = sum_i acc_i 2^(m_i - M) / L,
// lse = (M + log2 L) ln 2.  One 256-thread block per row: each group of D/4
// threads (a float4 each) takes every NG-th range, then the groups are summed
// in a fixed order, so the result is deterministic.
template <int D>
__global__ void __launch_bounds__(256)
rkv_reduce_kernel(const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int n_splits,
                  int64_t n_rows, float *__restrict__ o, float *__restrict__ lse)
{
    constexpr int TPC = D / 4;     // threads per copy of the row
    constexpr int NG = 256 / TPC;  // groups
    __shared__ float sM[256];
    __shared__ float4 sA[NG][TPC];
    __shared__ float sL[NG];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, grp = t / TPC, c = t - grp * TPC;
    float M = -INFINITY;
    for (int sp = t; sp < n_splits; sp += 256) M = fmaxf(M, part_ml[sp * n_rows + row].x);
    sM[t] = M;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (t < off) sM[t] = fmaxf(sM[t], sM[t + off]);
        __syncthreads();
    }
    M = sM[0];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll 4
    for (int sp = grp; sp < n_splits; sp += NG) {
        const float2 ml = part_ml[sp * n_rows + row];
        const float wgt = exp2f(ml.x - M);
        const float4 x = *(const float4 *)(part_acc + (sp * n_rows + row) * D + 4 * c);
        L = fmaf(ml.y, wgt, L);
        a.x = fmaf(x.x, wgt, a.x);
        a.y = fmaf(x.y, wgt, a.y);
        a.z = fmaf(x.z, wgt, a.z);
        a.w = fmaf(x.w, wgt, a.w);
    }
    sA[grp][c] = a;
    if (c == 0) sL[grp] = L;
    __syncthreads();
    if (grp == 0) {
        float4 s = sA[0][c];
        float Lt = sL[0];
        for (int gg = 1; gg < NG; ++gg) {
            s.x += sA[gg][c].x;
            s.y += sA[gg][c].y;
            s.z += sA[gg][c].z;
            s.w += sA[gg][c].w;
            Lt += sL[gg];
        }
        *(float4 *)(o + row * D + 4 * c) = make_float4(s.x / Lt, s.y / Lt, s.z / Lt, s.w / Lt);
        if (c == 0) lse[row] = (M + log2f(Lt)) * 0.69314718055994531f;
    }
}

hipError_t launch_reduce(int d, int64_t n_rows, int n_splits, const float *pa, const float2 *pm, float *o,
                         float *lse, hipStream_t s)
{
    const dim3 grid((unsigned)n_rows), block(256);
    switch (d) {
    case 64: hipLaunchKernelGGL(rkv_reduce_kernel<64>, grid, block, 0, s, pa, pm, n_splits, n_rows, o, lse); break;
    case 128: hipLaunchKernelGGL(rkv_reduce_kernel<128>, grid, block, 0, s, pa, pm, n_splits, n_rows, o, lse); break;
    case 256: hipLaunchKernelGGL(rkv_reduce_kernel<256>, grid, block, 0, s, pa, pm, n_splits, n_rows, o, lse); break;
    case 512: hipLaunchKernelGGL(rkv_reduce_kernel<512>, grid, block, 0, s, pa, pm, n_splits, n_rows, o, lse); break;
    default: return hipErrorInvalidValue;
    }
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

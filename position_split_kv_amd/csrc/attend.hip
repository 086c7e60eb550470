// attend.hip -- dispatch of the split kernel, and the fixed-order merge of
// the per-range partials into a segment's normalised output and LSE.
#include "common.h"

namespace rkv {

#define RKV_DECL(kt, vt)                                                                                  \
    hipError_t launch_split_k##kt##_v##vt(int d, int rt, dim3 grid, const float *q, const uint8_t *k,     \
                                          const uint8_t *v, float *pa, float2 *pm, const SplitParams &p,  \
                                          hipStream_t s);
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

hipError_t launch_split(int kt, int vt, int d, int rt, dim3 grid, const float *q, const uint8_t *k,
                        const uint8_t *v, float *pa, float2 *pm, const SplitParams &p, hipStream_t s)
{
#define RKV_CASE(kk, vv) \
    if (kt == kk && vt == vv) return launch_split_k##kk##_v##vv(d, rt, grid, q, k, v, pa, pm, p, s);
#define RKV_CASE_K(kk) RKV_CASE(kk, 0) RKV_CASE(kk, 1) RKV_CASE(kk, 2) RKV_CASE(kk, 3)
    RKV_CASE_K(0)
    RKV_CASE_K(1)
    RKV_CASE_K(2)
    RKV_CASE_K(3)
    return hipErrorInvalidValue;
}

// One wave per output row: M = max m_i, L = sum l_i 2^(m_i - M),
// o = sum acc_i 2^(m_i - M) / L, lse = (M + log2 L) ln 2.  Partials are in
// log2 units; the loop order over ranges is fixed.
template <int D>
__global__ void __launch_bounds__(64)
rkv_reduce_kernel(const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int n_splits,
                  int64_t n_rows, float *__restrict__ o, float *__restrict__ lse)
{
    constexpr int DPT = D / 64;
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    float M = -INFINITY;
    for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, part_ml[sp * n_rows + row].x);
    float L = 0.f, a[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) a[e] = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) {
        const float2 ml = part_ml[sp * n_rows + row];
        const float w = exp2f(ml.x - M);
        L = fmaf(ml.y, w, L);
        const float *src = part_acc + (sp * n_rows + row) * D + lane * DPT;
#pragma unroll
        for (int e = 0; e < DPT; ++e) a[e] = fmaf(src[e], w, a[e]);
    }
#pragma unroll
    for (int e = 0; e < DPT; ++e) o[row * D + lane * DPT + e] = a[e] / L;
    if (lane == 0) lse[row] = (M + log2f(L)) * 0.69314718055994531f;
}

hipError_t launch_reduce(int d, int64_t n_rows, int n_splits, const float *pa, const float2 *pm, float *o,
                         float *lse, hipStream_t s)
{
    const dim3 grid((unsigned)n_rows), block(64);
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

// combine.hip -- the segment merge ("F5 M7 -- Rolling KV", "Implementation
// decomposition, refined", S2): M = max_t lse_t, w_t = e^(lse_t - M),
// o = sum_t w_t o_t / sum_t w_t, lse = M + ln sum_t w_t, in F32.
#include "common.h"

namespace rkv {

// One block of 64 threads per row.  Every LSE of the row is read before any
// output is written, so o_out / lse_out may alias part 0.  The order of the
// sums over parts is fixed (deterministic), and a row whose only non-empty
// part is t gets w_t = 1 and w = 0 elsewhere, i.e. part t's bits.
__global__ void __launch_bounds__(64)
rkv_combine_kernel(CombineParts parts, int n_parts, int64_t n_rows, int d, float *o_out, float *lse_out)
{
    __shared__ float sw[kMaxParts];
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    float M = -INFINITY;
    for (int t = 0; t < n_parts; ++t) M = fmaxf(M, parts.lse[t][row]);
    if (lane < n_parts) sw[lane] = (M == -INFINITY) ? 0.f : expf(parts.lse[lane][row] - M);
    __syncthreads();
    float W = 0.f;
    for (int t = 0; t < n_parts; ++t) W += sw[t];
    for (int c = lane; c < d; c += 64) {
        float a = 0.f;
        for (int t = 0; t < n_parts; ++t) a = fmaf(sw[t], parts.o[t][row * d + c], a);
        o_out[row * d + c] = (M == -INFINITY) ? 0.f : a / W;
    }
    __syncthreads();
    if (lane == 0) lse_out[row] = (M == -INFINITY) ? -INFINITY : M + logf(W);
}

hipError_t launch_combine(int n_parts, const CombineParts &parts, int64_t n_rows, int d, float *o_out,
                          float *lse_out, hipStream_t s)
{
    hipLaunchKernelGGL(rkv_combine_kernel, dim3((unsigned)n_rows), dim3(64), 0, s, parts, n_parts, n_rows, d, o_out,
                       lse_out);
    return hipGetLastError();
}

}  // namespace rkv

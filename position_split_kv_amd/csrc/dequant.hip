// dequant.hip -- standalone q8_0 / q4_0 block dequantisation to binary32
// ("F5 M6 -- PolyKV", S0 and the tier-family table: 32 values per block,
// one binary16 scale d; q8_0 x = d*q, q4_0 x = d*(n-8) with element i < 16 in
// the low nibble of byte i and i >= 16 in the high nibble of byte i - 16).
// The binary32 products are exact.  Test and tooling utility only.
#include "common.h"

namespace rkv {

__device__ __forceinline__ float half_bits_to_float(uint32_t lo, uint32_t hi)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(lo | (hi << 8)));
}

__global__ void __launch_bounds__(256) rkv_dequant_q8_0_kernel(const uint8_t *__restrict__ b, int64_t n, float *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint8_t *blk = b + (i >> 5) * 34;
    const float d = half_bits_to_float(blk[0], blk[1]);
    out[i] = d * (float)(int8_t)blk[2 + (i & 31)];
}

__global__ void __launch_bounds__(256) rkv_dequant_q4_0_kernel(const uint8_t *__restrict__ b, int64_t n, float *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int j = (int)(i & 31);
    const uint8_t *blk = b + (i >> 5) * 18;
    const float d = half_bits_to_float(blk[0], blk[1]);
    const uint8_t byte = blk[2 + (j & 15)];
    const int code = j < 16 ? (byte & 15) : (byte >> 4);
    out[i] = d * (float)(code - 8);
}

hipError_t launch_dequant_q8_0(const void *blocks, int64_t n, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(rkv_dequant_q8_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)blocks, n, out);
    return hipGetLastError();
}

hipError_t launch_dequant_q4_0(const void *blocks, int64_t n, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(rkv_dequant_q4_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)blocks, n, out);
    return hipGetLastError();
}

}  // namespace rkv

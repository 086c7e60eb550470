// dequant.hip -- standalone q8_0 / q4_0 block dequantisation to binary32
// ("F5 M6 -- PolyKV", S0 and the tier-family table: 32 values per block,
// one binary16 scale d; q8_0 x = d*q, q4_0 x = d*(n-8) with element i < 16 in
// the low nibble of byte i and i >= 16 in the high nibble of byte i - 16).
// The binary32 products are exact.  Test and tooling utility only.
// Also the TBQ3 tier's inverse rotation (used on the output of attention over
// TBQ3 values) and its standalone dequantisation.
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

// ---- TBQ3 ("F5 M6 -- PolyKV", "S2 -- TurboQuant tier family"; layout and
// rotation in rkv.h)

struct Tbq3Args {
    float lv[4];
    uint32_t s1[4], s2[4];
};

__device__ __forceinline__ float sign_of(const uint32_t *mask, int i, float x)
{
    return ((mask[i >> 5] >> (i & 31)) & 1u) ? -x : x;
}

// x = S1 H S2 y / sqrt(128) for one 128-value block held by one wave, lane t
// holding values t (v0) and t + 64 (v1); H by its butterflies
// (w[i], w[i ^ h]) -> (w[i] + w[i ^ h], w[i ^ h] - w[i]) for the bit i & h.
__device__ __forceinline__ void inv_rotate128(float &v0, float &v1, int t, const Tbq3Args &a)
{
    v0 = sign_of(a.s2, t, v0);
    v1 = sign_of(a.s2, t + 64, v1);
    const float x = v0 + v1, y = v0 - v1;  // h = 64: the two halves
    v0 = x;
    v1 = y;
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) {
        const float p0 = __shfl_xor(v0, h, 64), p1 = __shfl_xor(v1, h, 64);
        v0 = (t & h) ? p0 - v0 : v0 + p0;
        v1 = (t & h) ? p1 - v1 : v1 + p1;
    }
    constexpr float kInvSqrt128 = 0.088388347648318440550f;  // 1 / sqrt(128)
    v0 = sign_of(a.s1, t, v0) * kInvSqrt128;
    v1 = sign_of(a.s1, t + 64, v1) * kInvSqrt128;
}

// Rotated value i of a TBQ3 block: (-1)^sign c_m n / sqrt(128).
__device__ __forceinline__ float tbq3_rotated(const uint8_t *blk, int i, float n, const Tbq3Args &a)
{
    const int m = (blk[4 + (i >> 2)] >> (2 * (i & 3))) & 3;
    const float c = m == 0 ? a.lv[0] : m == 1 ? a.lv[1] : m == 2 ? a.lv[2] : a.lv[3];
    const float y = c * n * 0.088388347648318440550f;
    return ((blk[36 + (i >> 3)] >> (i & 7)) & 1) ? -y : y;
}

// One wave per block.
__global__ void __launch_bounds__(64) rkv_dequant_tbq3_kernel(const uint8_t *__restrict__ b, float *__restrict__ out,
                                                              const Tbq3Args a)
{
    const int t = threadIdx.x;
    const uint8_t *blk = b + (int64_t)blockIdx.x * 52;
    const float n = half_bits_to_float(blk[0], blk[1]);
    float v0 = tbq3_rotated(blk, t, n, a), v1 = tbq3_rotated(blk, t + 64, n, a);
    inv_rotate128(v0, v1, t, a);
    out[(int64_t)blockIdx.x * 128 + t] = v0;
    out[(int64_t)blockIdx.x * 128 + t + 64] = v1;
}

// One wave per (row, 128-value block) of o, in place.
__global__ void __launch_bounds__(64) rkv_unrotate_kernel(float *__restrict__ o, const Tbq3Args a)
{
    const int t = threadIdx.x;
    float *p = o + (int64_t)blockIdx.x * 128;
    float v0 = p[t], v1 = p[t + 64];
    inv_rotate128(v0, v1, t, a);
    p[t] = v0;
    p[t + 64] = v1;
}

static Tbq3Args args_of(const Tbq3Consts &c)
{
    Tbq3Args a;
    for (int i = 0; i < 4; ++i) {
        a.lv[i] = c.lv[i];
        a.s1[i] = c.s1[i];
        a.s2[i] = c.s2[i];
    }
    return a;
}

hipError_t launch_dequant_tbq3(const void *blocks, int64_t n, float *out, const Tbq3Consts &c, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rkv_dequant_tbq3_kernel, dim3((unsigned)(n / 128)), dim3(64), 0, s, (const uint8_t *)blocks,
                       out, args_of(c));
    return hipGetLastError();
}

hipError_t launch_unrotate(float *o, int64_t n_rows, int d, const Tbq3Consts &c, hipStream_t s)
{
    const int64_t nb = n_rows * (d / 128);
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(rkv_unrotate_kernel, dim3((unsigned)nb), dim3(64), 0, s, o, args_of(c));
    return hipGetLastError();
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

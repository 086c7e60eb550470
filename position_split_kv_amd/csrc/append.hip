// append.hip -- the KV write path: new binary32 K / V rows stored at their
// positions in a layer's window or tail, in each region's storage type.
//
// Routing ("Rolling-KV: step/graph-level tail prefetch (design)", section
// "Staged plan", S0 / bug-1341; "F5 M7 -- Rolling KV", section "2026-07-14 --
// bug-2172 SHIPPED"): per layer, a row at position p goes to window row p when
// p < wc, else to tail row p - wc.  The host cuts the call's consecutive
// positions into at most three destination ranges (window, tail, and the
// optional device copy of the tail rows); the kernel only stores.
//
// Storage (the block formats of "F5 M6 -- PolyKV", section "S0 -- Bootstrap";
// the pages give no rule for making codes, the one taken is the common rule
// for the formats, computed in binary32 with no fused multiply-add):
//   f32   the value;  f16  nearest binary16, ties to even;
//   q8_0  d = amax / 127, q = round-half-away(x * (1/d));
//   q4_0  m = first value of largest magnitude (+0 for zeros), d = m / -8,
//         n = min(15, trunc(x * (1/d) + 8.5));
//   1/d = 0 when d = 0; the scale is stored as the nearest binary16 of the
//   binary32 d, the codes come from the binary32 d.
//
// Workgroups of 4 waves; each wave stores whole (token, KV head) rows in
// turn: it reads the K row and the V row (D binary32 values, coalesced) and,
// for every destination the token has, encodes each row in registers and
// stores it from there (bytes for codes, 16 bits for scales and binary16
// values, 32 bits for binary32 values on 4-byte aligned rows).  Lane l holds values
// l + 64 i, so a 32-value block is one half-wave and its reductions are
// xor-shuffles within the half.  HBM-bound for long appends (4 B read per
// value, row bytes written per destination), latency-bound for one token.
#include "common.h"

namespace rkv {

namespace {

// amax over the 32 lanes of a half-wave.
__device__ __forceinline__ float half_max(float a)
{
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    return a;
}

__device__ __forceinline__ uint16_t f16_bits(float x)
{
    const _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Encode one row (values xr[i] = x[lane + 64 i]) of type t and store it at
// row (global memory, 2-byte aligned): each lane stores its own values, codes
// and (lane 0 of a block) scale with 1-, 2- or 4-byte stores; the stores of a
// wave cover the row's bytes contiguously.
template <int D>
__device__ __forceinline__ void encode_row(int t, const float (&xr)[D / 64], uint8_t *row)
{
    // the code decisions are defined on separately rounded binary32 products
    // and sums: no multiply-add contraction here
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63, e = lane & 31;
    if (t == kF32) {
        if (((uintptr_t)row & 3) == 0) {
#pragma unroll
            for (int i = 0; i < D / 64; ++i) ((float *)row)[lane + 64 * i] = xr[i];
        } else {
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const uint32_t b = __float_as_uint(xr[i]);
                ((uint16_t *)row)[2 * (lane + 64 * i)] = (uint16_t)b;
                ((uint16_t *)row)[2 * (lane + 64 * i) + 1] = (uint16_t)(b >> 16);
            }
        }
    } else if (t == kF16) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) ((uint16_t *)row)[lane + 64 * i] = f16_bits(xr[i]);
    } else if (t == kQ8) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int blk = 2 * i + (lane >> 5);
            const float x = xr[i];
            const float amax = half_max(fabsf(x));
            const float d = amax / 127.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            const float v = x * id;
            row[34 * blk + 2 + e] = (uint8_t)(int8_t)(int)roundf(v);
            if (e == 0) *(uint16_t *)(row + 34 * blk) = f16_bits(d);
        }
    } else {  // kQ4
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int blk = 2 * i + (lane >> 5);
            const float x = xr[i];
            // largest magnitude, first index among equals: the key orders by
            // |x| (its bits order like the value for |x| >= 0), then by 31 - e
            const uint32_t ab = __float_as_uint(fabsf(x));
            uint32_t kh = ab, kl = 31u - (uint32_t)e;
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) {
                const uint32_t oh = __shfl_xor(kh, o, 64), ol = __shfl_xor(kl, o, 64);
                if (oh > kh || (oh == kh && ol > kl)) {
                    kh = oh;
                    kl = ol;
                }
            }
            const int src = (lane & 32) + 31 - (int)kl;
            const float xm = __shfl(x, src, 64);
            const float m = kh == 0u ? 0.0f : xm;
            const float d = m / -8.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            const float v = x * id;
            const float w = v + 8.5f;
            const int c = min((int)w, 15);
            const int hi = __shfl(c, lane + 16, 64);  // n[e + 16] for e < 16
            if (e < 16) row[18 * blk + 2 + e] = (uint8_t)(c | (hi << 4));
            if (e == 0) *(uint16_t *)(row + 18 * blk) = f16_bits(d);
        }
    }
}

constexpr int kAppendWaves = 4;  // waves per workgroup; each wave stores whole rows

template <int D>
__global__ void __launch_bounds__(64 * kAppendWaves) rkv_append_kernel(const float *__restrict__ k_new,
                                                                       const float *__restrict__ v_new,
                                                                       AppendParams p, int n_rows)
{
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    // row r = (token, KV head) = (r / n_kv_heads, r % n_kv_heads); the waves of
    // the grid take rows in turn (a wave-uniform loop: no workgroup barriers)
    for (int r = blockIdx.x * kAppendWaves + wv; r < n_rows; r += gridDim.x * kAppendWaves) {
        const int tok = r / p.n_kv_heads, h = r - tok * p.n_kv_heads;
        const int64_t src = (int64_t)r * D;
        float xk[D / 64], xv[D / 64];
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            xk[i] = k_new[src + lane + 64 * i];
            xv[i] = v_new[src + lane + 64 * i];
        }
        for (int di = 0; di < p.n_dst; ++di) {
            const AppendDst &dd = p.dst[di];
            if (tok < dd.first_tok || tok >= dd.first_tok + dd.n_tok) continue;  // uniform over the wave
            const int64_t rr = dd.row0 + (tok - dd.first_tok);
            encode_row<D>(dd.k_type, xk, dd.k + rr * dd.k_pos + h * dd.k_head);
            encode_row<D>(dd.v_type, xv, dd.v + rr * dd.v_pos + h * dd.v_head);
        }
    }
    // rows written to host memory reach it before the kernel ends (a copy
    // engine reads them next, ordered only through a host-visible signal)
    if (p.sys_fence) __threadfence_system();
}

}  // namespace

hipError_t launch_append(int d, int n_tokens, int n_kv_heads, const float *k_new, const float *v_new,
                         const AppendParams &p, hipStream_t stream)
{
    if (n_tokens <= 0) return hipSuccess;
    const int64_t n_rows = (int64_t)n_tokens * n_kv_heads;
    if (n_rows > 0x7fffffff - 64 * kAppendWaves) return hipErrorInvalidValue;
    // one row per wave up to 8192 workgroups (rows in flight hide the load
    // latency of each row), then waves take several rows
    const int64_t need = (n_rows + kAppendWaves - 1) / kAppendWaves;
    const dim3 grid((unsigned)(need < 8192 ? need : 8192)), block(64 * kAppendWaves);
    const int nr = (int)n_rows;
    switch (d) {
    case 64: hipLaunchKernelGGL(rkv_append_kernel<64>, grid, block, 0, stream, k_new, v_new, p, nr); break;
    case 128: hipLaunchKernelGGL(rkv_append_kernel<128>, grid, block, 0, stream, k_new, v_new, p, nr); break;
    case 256: hipLaunchKernelGGL(rkv_append_kernel<256>, grid, block, 0, stream, k_new, v_new, p, nr); break;
    case 512: hipLaunchKernelGGL(rkv_append_kernel<512>, grid, block, 0, stream, k_new, v_new, p, nr); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rkv

// probe.hip -- a plain streaming-read kernel, the measured read ceiling that
// the attention kernels are reported against (librkvprobe.so, loaded by
// bench.py).  Not part of the attention library or its ABI.
//
// Each launch reads up to two byte ranges once, front to back, with 16-byte
// non-temporal vector loads (the cache policy of the attention kernel's K
// tiles): thread t of the grid takes the 16-byte chunks t, t + T, t + 2T, ...
// (T = threads in the grid), eight loads in flight per thread, so every
// wavefront load covers 1 KiB of consecutive bytes.  The chunks are folded
// with xor into one word per thread, stored only if it equals a constant the
// data practically never produces (the loads cannot be removed, and the
// kernel writes nothing in practice).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

__device__ __forceinline__ uint32_t read_range(const u32x4 *__restrict__ p, uint64_t n, uint64_t t, uint64_t T)
{
    uint32_t acc = 0;
    uint64_t i = t;
    for (; i + 7 * T < n; i += 8 * T) {
        u32x4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(p + i + u * T);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= fold(x[u]);
    }
    for (; i < n; i += T) acc ^= fold(__builtin_nontemporal_load(p + i));
    return acc;
}

__global__ void __launch_bounds__(256) rkv_probe_read_kernel(const u32x4 *__restrict__ a, uint64_t na,
                                                             const u32x4 *__restrict__ b, uint64_t nb,
                                                             uint32_t *__restrict__ sink)
{
    const uint64_t T = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t acc = read_range(a, na, t, T) ^ read_range(b, nb, t, T);
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read [a, a + a_bytes) and [b, b + b_bytes) once (device memory, 16-byte
// aligned, sizes multiples of 16; b may be NULL with b_bytes 0) with `blocks`
// workgroups of 256 threads.  sink: device memory of `blocks` words (written
// only in the practically impossible case above).  Returns the hipError_t of
// the launch (0 on success), -1 for bad arguments.
int rkv_probe_read(const void *a, uint64_t a_bytes, const void *b, uint64_t b_bytes, int blocks, void *sink,
                   hipStream_t stream)
{
    if (!a || (b_bytes && !b) || !sink || blocks < 1 || (a_bytes | b_bytes) % 16 || ((uintptr_t)a | (uintptr_t)b) % 16)
        return -1;
    hipLaunchKernelGGL(rkv_probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4 *)a,
                       a_bytes / 16, (const u32x4 *)b, b_bytes / 16, (uint32_t *)sink);
    return (int)hipGetLastError();
}

}  // extern "C"

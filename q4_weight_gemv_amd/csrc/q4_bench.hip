// Streaming-read kernel used as the measured HBM ceiling beside the products.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q4_bench.h"
#include "q4_internal.h"

namespace q4 {
namespace bench {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *sink)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256u;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256u + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    // Four independent loads per iteration keep enough requests in flight.
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a ^ b) ^ (c ^ d);
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (!sink) {
        // A pure read: the fold is consumed here (so the loads stay) and
        // nothing is stored or exchanged.
        asm volatile("" ::"v"(v));
        return;
    }
    // Each wave's fold of everything it read, one plain store per wave (no
    // barrier holds a finished wave, no shared word serializes them).
    for (int o = 32; o > 0; o >>= 1) v ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o));
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4u + (threadIdx.x >> 6)] = v;
}

}  // namespace bench
}  // namespace q4

extern "C" int q4_read_probe(const void *p, size_t bytes, uint32_t *sink, int groups, void *hip_stream)
{
    if (!p || bytes == 0 || groups < 1 || groups > 65536) return Q4_EINVAL;
    if ((bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return Q4_EALIGN;
    hipLaunchKernelGGL(q4::bench::read_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const q4::bench::u32x4 *>(p),
                       static_cast<uint64_t>(bytes / 16), sink);
    return q4::hip_status(hipGetLastError());
}

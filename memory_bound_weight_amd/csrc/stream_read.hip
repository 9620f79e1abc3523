// Read-only streaming pass over a buffer: the achievable-bandwidth ceiling a
// product kernel is measured against (llm-rs design post, section 6: measure
// against a ceiling).  Same access shape as the products at their best: short
// wavefronts, each issuing four 16-byte loads per lane (4 KB) at once.
#include "registry.h"

namespace lin {

__device__ uint32_t g_read_sink;   // written only if the xor of the data hits a fixed value

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16) {
    constexpr int U = 4;
    const size_t wave = (size_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    const size_t lane = threadIdx.x & 63;
    const size_t base = wave * (kWave * U);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + u * kWave + lane;
        v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    if (acc == 0x9E3779B9u) g_read_sink = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t per_block = (size_t)kBlock * 4;   // 16-byte words per workgroup
    const u32x4* p = (const u32x4*)buf;
    void* args[] = {(void*)&p, (void*)&n16};
    return hipLaunchKernel((const void*)&stream_read_kernel, dim3((unsigned)((n16 + per_block - 1) / per_block)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace lin

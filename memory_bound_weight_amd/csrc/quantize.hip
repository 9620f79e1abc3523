// Load-time weight preparation for the int4-g64 format (tinyinfer post, TL;DR:
// 4-bit weights plus one fp16 scale per 64) and for INT8 with one fp32 scale
// per output channel (TileInfer.jl post, INT8 section), and the cache-flush
// kernel used while tuning (a read sweep over a buffer larger than the caches).
//
// One thread per (row, group of 64): a = max |w|; s = fp16 nearest to a/7
// (ties to even, saturated at 65504); q = s > 0 ? clamp(rint(w/s), -8, 7) : 0
// with a/7 and w/s in fp64, so both roundings happen exactly once.  Two codes
// per byte along k, even k in the low nibble, 4-bit two's complement.
#include "registry.h"

namespace lin {

// Exact value of a bf16 / fp16 bit pattern, assembled bit by bit so that no
// hardware denormal mode is involved (finite inputs).
__device__ __forceinline__ double bf16_to_f64(uint32_t h) {
    const uint64_t sign = (uint64_t)(h >> 15) << 63;
    const uint32_t e = (h >> 7) & 0xFF, f = h & 0x7F;
    if (e == 0)   // zero or subnormal: f * 2^-133
        return __builtin_bit_cast(double, sign | __builtin_bit_cast(uint64_t, (double)f * 0x1p-133));
    return __builtin_bit_cast(double, sign | ((uint64_t)(e - 127 + 1023) << 52) | ((uint64_t)f << 45));
}

// Nearest binary16 to a finite, non-negative double (round half to even),
// from the bit layout: keep 10 fraction bits (normal) or align to 2^-24
// (subnormal) and round on the discarded bits.
__device__ uint32_t f64_to_f16_rne(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    if (b == 0) return 0;
    const int e = (int)(b >> 52) - 1023;
    if (e >= 16) return 0x7C00;
    const uint64_t mant = (b & ((1ull << 52) - 1)) | (1ull << 52);
    const int shift = (e >= -14) ? 42 : (28 - e);
    if (shift > 63) return 0;
    uint64_t q = mant >> shift;
    const uint64_t rem = mant & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (e >= -14) {
        int E = e;
        if (q == 2048) { q = 1024; ++E; }
        if (E + 15 >= 31) return 0x7C00;
        return (uint32_t)(((E + 15) << 10) | (int)(q - 1024));
    }
    return (uint32_t)q;   // subnormal; 1024 encodes the smallest normal
}

__device__ __forceinline__ double f16_to_f64(uint32_t h) {   // h non-negative, finite
    const uint32_t e = (h >> 10) & 0x1F, f = h & 0x3FF;
    if (e == 0) return (double)f * 0x1p-24;
    return __builtin_bit_cast(double, ((uint64_t)(e - 15 + 1023) << 52) | ((uint64_t)f << 42));
}

__global__ __launch_bounds__(256) void quantize_q4g64_kernel(const uint16_t* __restrict__ W,
                                                             uint8_t* __restrict__ Wq,
                                                             uint16_t* __restrict__ S,
                                                             int N, int K) {
    const int G = K >> 6;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)N * G) return;
    const int64_t n = t / G;
    const int g = (int)(t - n * G);
    const u32x4* src = (const u32x4*)(W + n * (int64_t)K + (int64_t)g * 64);
    u32x4 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_nontemporal_load(src + i);
    uint32_t amax = 0;   // |w| as bf16 bits: ordering of magnitudes = integer ordering
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = w[i][j] & 0x7FFFu, hi = (w[i][j] >> 16) & 0x7FFFu;
            amax = max(amax, max(lo, hi));
        }
    uint32_t sb = f64_to_f16_rne(bf16_to_f64(amax) / 7.0);
    if (sb == 0x7C00) sb = 0x7BFF;
    S[n * (int64_t)G + g] = (uint16_t)sb;
    const double s = f16_to_f64(sb);
    u32x4 packed[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;   // 8 codes of w[i]: k = 8i .. 8i+7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t bits = h ? (w[i][j] >> 16) : (w[i][j] & 0xFFFFu);
                int q = 0;
                if (s > 0.0) {
                    double r = __builtin_rint(bf16_to_f64(bits) / s);
                    r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
                    q = (int)r;
                }
                word |= (uint32_t)(q & 0xF) << (4 * (2 * j + h));
            }
        }
        packed[i >> 2][i & 3] = word;
    }
    u32x4* dst = (u32x4*)(Wq + n * (int64_t)(K / 2) + (int64_t)g * 32);
    dst[0] = packed[0];
    dst[1] = packed[1];
}

hipError_t launch_quantize_q4g64(const void* W, void* Wq, void* S, int N, int K, hipStream_t stream) {
    const int64_t groups = (int64_t)N * (K / 64);
    if (groups == 0) return hipSuccess;
    const dim3 grid((unsigned)((groups + 255) / 256));
    const uint16_t* w = (const uint16_t*)W;
    uint8_t* wq = (uint8_t*)Wq;
    uint16_t* s = (uint16_t*)S;
    void* args[] = {(void*)&w, (void*)&wq, (void*)&s, (void*)&N, (void*)&K};
    return hipLaunchKernel((const void*)&quantize_q4g64_kernel, grid, dim3(256), args, 0, stream);
}

// INT8 with one fp32 scale per output channel, one workgroup per row:
// a = max |w| over the row; s = fp32 nearest to a / 127 (the quotient formed in
// fp64, then rounded once to fp32); q = s > 0 ? clamp(rint(w / s), -127, 127) : 0
// with w / s in fp64 (TileInfer.jl post, INT8 section: scale = max|x| / 127,
// every entry rounded to the nearest multiple of the scale).

__global__ __launch_bounds__(256) void quantize_i8_kernel(const uint16_t* __restrict__ W,
                                                          int8_t* __restrict__ Wq,
                                                          float* __restrict__ S, int K) {
    const int64_t n = blockIdx.x;
    const uint16_t* row = W + n * (int64_t)K;
    const int nun = K >> 3;   // 16-byte units of 8 weights
    uint32_t amax = 0;        // |w| as bf16 bits: magnitude order = integer order
    for (int i = threadIdx.x; i < nun; i += 256) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)row + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = max(amax, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    const float s = (float)(bf16_to_f64(red[0]) / 127.0);
    if (threadIdx.x == 0) S[n] = s;
    const double sd = (double)s;
    for (int i = threadIdx.x; i < nun; i += 256) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)row + i);
        uint32_t out[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int q = 0;
                if (s > 0.f) {
                    double r = __builtin_rint(bf16_to_f64(h ? (v[j] >> 16) : (v[j] & 0xFFFFu)) / sd);
                    r = r < -127.0 ? -127.0 : (r > 127.0 ? 127.0 : r);
                    q = (int)r;
                }
                out[j >> 1] |= (uint32_t)(q & 0xFF) << (8 * (2 * (j & 1) + h));
            }
        *(uint2*)(Wq + n * (int64_t)K + 8 * i) = make_uint2(out[0], out[1]);
    }
}

hipError_t launch_quantize_i8(const void* W, void* Wq, void* S, int N, int K, hipStream_t stream) {
    if (N == 0 || K == 0) return hipSuccess;
    const uint16_t* w = (const uint16_t*)W;
    int8_t* wq = (int8_t*)Wq;
    float* s = (float*)S;
    void* args[] = {(void*)&w, (void*)&wq, (void*)&s, (void*)&K};
    return hipLaunchKernel((const void*)&quantize_i8_kernel, dim3((unsigned)N), dim3(256), args, 0, stream);
}


// Reads (does not write) the buffer: the caches end up full of clean lines, as
// after other kernels' reads, with no dirty data whose write-back would slow
// the timed call.  The store below only keeps the loads alive.
__global__ __launch_bounds__(256) void flush_kernel(u32x4* buf, size_t n16, uint32_t salt) {
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (size_t i = i0; i < n16; i += (size_t)gridDim.x * blockDim.x) {
        const u32x4 v = buf[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == salt && i0 < n16) buf[i0] = u32x4{acc, acc, acc, acc};
}

hipError_t launch_flush(void* buf, size_t n16, uint32_t salt, hipStream_t stream) {
    u32x4* b = (u32x4*)buf;
    void* args[] = {(void*)&b, (void*)&n16, (void*)&salt};
    return hipLaunchKernel((const void*)&flush_kernel, dim3(4096), dim3(256), args, 0, stream);
}

}  // namespace lin

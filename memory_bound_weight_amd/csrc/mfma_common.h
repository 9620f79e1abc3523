// Pieces shared by the matrix-core ring kernels: the scalar-base form of the
// direct-to-LDS load, the 16x16x32 bf16 product and the store of a
// wavefront's output tiles (direct, or split-K through the workspace with a
// deterministic reduction).
#pragma once

#include "kern_common.h"

namespace lin {

// dma16 with a wavefront-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the saddr form of global_load_lds_dwordx4): moving to the next
// block is a scalar add, with no per-lane address arithmetic.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved: set here, used by nothing else
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, const void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(LDS_AS const void*)lds;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(l)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// A pointer every lane of the wavefront holds the same value of, as such.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D = A . B + C for A 16x32 (lane l: row l mod 16, k 8 (l / 16) .. + 7), B 32x16
// (lane l: column l mod 16, the same k), C and D 16x16 fp32 (lane l: column
// l mod 16, rows 4 (l / 16) .. + 3).
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt with vmcnt <= V (V < 64; 63 does not wait on loads) and
// lgkmcnt <= G (G < 16); expcnt not waited on.
template <int V, int G>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(V >= 0 && V < 64 && G >= 0 && G < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (G << 8));
}

// Wait (also for every LDS access) until the loads of the current ring stage
// have landed while `after` later stages, L loads each, may still be in
// flight: loads are issued in stage order and complete in order.
template <int L, int D, int J = 0>
__device__ __forceinline__ void wait_stages(int after) {
    if constexpr (J <= D - 2) {
        if (after == J) {
            wait_vm_lgkm<J * L, 0>();
            return;
        }
        wait_stages<L, D, J + 1>(after);
    } else {
        wait_vm_lgkm<0, 0>();
    }
}

// Workgroup barrier that the compiler may not move memory accesses across
// (a bare s_barrier: __syncthreads would also wait for the loads in flight).
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Store the NF x MT 16x16 accumulators of one wavefront: lane l holds W row
// n_tile * BN + nl0 + 16 f + l mod 16 and tokens m_tile * TM + ml0 + 16 t +
// 4 (l / 16) + r.  S == 1 writes Y directly.  Otherwise the partial tile goes
// to the workspace with coherent (agent-scope) stores, the tile is counted,
// and the workgroup that completes the count adds the S partials in split
// order (deterministic) and resets the counter.  Partial element (m, n) of a
// tile sits at m * BN + n (tile-local).  The partials are written and read
// with agent-scope atomic accesses, which go to the device-coherent level
// directly, so publishing needs no L2 write-back and reading no L2 invalidate
// (whole-cache operations on this chip that cost more than the product).
// Ordering without acquire/release: the partial stores bypass the per-XCD L2s
// and s_waitcnt(0) returns only once the coherence point has acknowledged
// them; the barrier then keeps the counter increment (and the compiler) after
// them.  The workgroup whose increment returns S - 1 therefore runs after
// every other workgroup's partials are visible at that point, and reads them
// with agent-scope loads, which do not hit a stale L2 line.
// Every thread of the workgroup must call this (it contains workgroup
// barriers when S > 1).
template <int BN, int TM, int NF, int MT>
__device__ __forceinline__ void store_tiles(const f32x4 (&acc)[NF][MT], const KArgs& a, int S,
                                            int n_tile, int m_tile, int ks, int n_tiles,
                                            int m_tiles, int nl0, int ml0) {
    const int M = a.M, N = a.N;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = n_tile * BN + nl0;
    const int m0 = m_tile * TM + ml0;
    if (S == 1) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int n = n0 + f * 16 + l16;
            if (n >= N) continue;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + t * 16 + lg * 4 + r;
                    if (m < M) a.Y[(int64_t)m * N + n] = acc[f][t][r];
                }
        }
        return;
    }
    const int tiles = m_tiles * n_tiles;
    const int tile = n_tile * m_tiles + m_tile;
    uint32_t* cnt = (uint32_t*)a.ws;
    float* parts = (float*)((uint8_t*)a.ws + ws_counter_bytes(tiles));
    const size_t tile_elems = (size_t)TM * BN;
    float* mine = parts + ((size_t)ks * tiles + tile) * tile_elems;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(&mine[(size_t)(ml0 + t * 16 + lg * 4 + r) * BN + nl0 + f * 16 + l16],
                                   acc[f][t][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);   // the partial stores are complete
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last = (old == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int n = n0 + f * 16 + l16;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t e = (size_t)(ml0 + t * 16 + lg * 4 + r) * BN + nl0 + f * 16 + l16;
                float v = 0.f;
                for (int j = 0; j < S; ++j)
                    v += __hip_atomic_load(&parts[((size_t)j * tiles + tile) * tile_elems + e],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int m = m0 + t * 16 + lg * 4 + r;
                if (m < M && n < N) a.Y[(int64_t)m * N + n] = v;
            }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lin

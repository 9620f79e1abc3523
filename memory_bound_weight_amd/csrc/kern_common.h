// Device helpers shared by the gfx950 kernels of the linear-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lin {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Arguments common to every product kernel (passed by value).
struct KArgs {
    const void* W;   // bf16 [N][K] or packed int4 [N][K/2]
    const void* S;   // fp16 [N][K/64] scales (int4 only)
    const void* X;   // bf16 [M][K]
    float* Y;        // fp32 [M][N]
    int M, N, K;
    int splits;      // split-K factor (matrix-core path), 1 otherwise
    void* ws;        // split-K workspace: tile counters, then partial tiles
    const float* R;  // residual fp32 [M][N] of the add epilogue (may equal Y)
    const void* G;   // bf16 [K] gain of the RMSNorm prologue
    float eps;       // RMSNorm: added to the mean square
};

// Epilogues of the batch-1 products (the values of lin_epilogue).
constexpr int kEpiNone = 0, kEpiAdd = 1, kEpiSwiglu = 2;

// silu(g) * u, silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

constexpr int kWave = 64;
constexpr int kBlock = 256;   // four wavefronts per workgroup

// Index of this wavefront in its workgroup, as a wave-uniform (scalar) value so
// that row addresses derived from it live in SGPRs.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Weights are read exactly once per call: a non-temporal 16-byte load keeps
// them from displacing the activations, which every wavefront re-reads.
// Addresses are a wave-uniform base plus a 32-bit per-lane byte offset, which
// maps to the scalar-base form of the global load (no 64-bit vector adds).
__device__ __forceinline__ u32x4 load_w16(const uint8_t* base, uint32_t off) {
    return __builtin_nontemporal_load((const u32x4*)(base + off));
}
__device__ __forceinline__ u32x4 load_x16(const uint8_t* base, uint32_t off) {
    return *(const u32x4*)(base + off);
}
__device__ __forceinline__ uint16_t load_w2(const uint8_t* base, uint32_t off) {
    return __builtin_nontemporal_load((const uint16_t*)(base + off));
}

// s_waitcnt with vmcnt <= VM and lgkmcnt <= LGKM (expcnt not waited on).
// The empty asm statements keep memory accesses from moving across it.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_cnt() {
    static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier without the vmcnt(0) that __syncthreads adds: loads still
// in flight stay in flight.  Callers wait for what the barrier must cover.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

#define LDS_AS __attribute__((address_space(3)))

// One direct-to-LDS load (gfx950 global_load_lds_dwordx4): 16 bytes per lane
// from `g` into LDS at the wavefront-uniform address `lds` + 16 * lane.
// Written as inline assembly so that the compiler does not make later LDS
// reads wait for every outstanding load; callers order it with wait_cnt and
// barriers.  M0 is set here and used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved: set here, used by nothing else
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(LDS_AS const void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

namespace {
// Lanes with nothing to load read these zeros (a valid address).
__device__ __attribute__((aligned(16))) const u32x4 g_zero16 = {0u, 0u, 0u, 0u};
}  // namespace

// 16-byte units of LDS that stage_x_dma fills for MT token rows of K bf16:
// MT * K / 8, rounded up to whole wavefront loads (64 units).
__host__ __device__ inline size_t stage_x_units(int MT, int K) {
    return ((size_t)MT * (size_t)(K / 8) + 63) / 64 * 64;
}

// Issue the direct-to-LDS loads of MT token rows of x (bf16 [M][K], K a
// multiple of 8) into `dst` in natural order, dst[m * K / 8 + j] = 16-byte
// unit j of row m.  Rows m >= M load row 0 (finite values, never stored).
// Wavefront loads are dealt round-robin to the four wavefronts; units past
// the end land in the padding of stage_x_units.  Returns without waiting:
// the loads complete in issue order with the wavefront's other loads.
__device__ __forceinline__ void stage_x_dma(const void* X, int M, int MT, int K, u32x4* dst) {
    const int nch = K >> 3;
    const int total = MT * nch;
    const int nload = (total + 63) >> 6;
    const int lane = threadIdx.x & 63;
    const u32x4* src = (const u32x4*)X;
    for (int i = wave_id(); i < nload; i += 4) {
        const int u = i * 64 + lane;
        const u32x4* p = &g_zero16;
        if (u < total) {
            const int m = u / nch;
            p = src + (m < M ? u : u - m * nch);
        }
        dma16(p, dst + i * 64);
    }
}

// acc + a.lo*b.lo + a.hi*b.hi on two bf16 pairs (v_dot2_f32_bf16); the
// bf16 x bf16 products are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// int4 codes as exact bf16 values.  Flipping bit 3 of a 4-bit two's
// complement code q gives n = q + 8 in [0, 15]; placed in the top four mantissa
// bits of a bf16 whose exponent is 4 (value 16), the pattern reads 16 + n =
// 24 + q exactly.  (w >> s) & 0x00780078 ^ 0x41C041C0 does this for the
// nibbles at bits 3 + s .. 6 + s and 19 + s .. 22 + s of w with one 3-input
// bitwise operation (v_bitop3_b32): two codes per dword, each exact in the
// products with bf16 x.  The products then carry 24 sum x, removed in fp32;
// the offset of 24 code steps (the smallest that keeps every code's exponent
// equal) bounds the rounding that removal adds.
constexpr uint32_t kQ4Mask = 0x00780078u, kQ4Code = 0x41C041C0u;
constexpr float kQ4Offset = 24.f;
constexpr uint32_t kQ4NegOffsetPair = 0xC1C0C1C0u;   // bf16 pair (-24, -24)

template <int S>
__device__ __forceinline__ uint64_t q4_shr64(uint64_t v) {
    uint64_t r;
    asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "I"(S), "v"(v));
    return r;
}
template <int S>
__device__ __forceinline__ uint64_t q4_shl64(uint64_t v) {
    uint64_t r;
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "I"(S), "v"(v));
    return r;
}

// Codes of two dwords lo = (uint32_t)w, hi = w >> 32, whose nibble i sits at
// bits 4i .. 4i + 3.  o[i] (i < 4) pairs nibble i of lo with nibble i + 4 of lo
// (low and high bf16 halves), o[4 + i] the same for hi.  Every dword needs
// nibble i moved to bit 3 (a shift right by 4i - 3, left by 3 for i = 0); the
// shifts act on both dwords at once with 64-bit shifts, and the bits that cross
// from one dword into the other land outside the mask.  12 operations for 16
// codes.
__device__ __forceinline__ void q4_unpack2(uint64_t w, uint32_t (&o)[8]) {
    const uint64_t t0 = q4_shl64<3>(w), t1 = q4_shr64<1>(w), t2 = q4_shr64<5>(w),
                   t3 = q4_shr64<9>(w);
    o[0] = ((uint32_t)t0 & kQ4Mask) ^ kQ4Code;
    o[1] = ((uint32_t)t1 & kQ4Mask) ^ kQ4Code;
    o[2] = ((uint32_t)t2 & kQ4Mask) ^ kQ4Code;
    o[3] = ((uint32_t)t3 & kQ4Mask) ^ kQ4Code;
    o[4] = ((uint32_t)(t0 >> 32) & kQ4Mask) ^ kQ4Code;
    o[5] = ((uint32_t)(t1 >> 32) & kQ4Mask) ^ kQ4Code;
    o[6] = ((uint32_t)(t2 >> 32) & kQ4Mask) ^ kQ4Code;
    o[7] = ((uint32_t)(t3 >> 32) & kQ4Mask) ^ kQ4Code;
}

__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return bitsf((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(v), CTRL, 0xF, 0xF, false));
}

// Sum each of V per-lane values over the 64 lanes of a wavefront, V a power of
// two <= 64.  Lane pairs l, l^32 and then l, l^16 are combined with the gfx950
// permlane32/permlane16 swaps, which exchange half of the values in one
// instruction, so V values cost about 2.5 V operations instead of 6 V.  The
// rest is summed inside rows of 16 lanes with DPP.  Every lane must be active.
//
// On return, slot j < reduce_slots(V) of lane l holds the total of value index
// reduce_index<V>(j, l); lanes of one 16-lane row hold the same totals.
constexpr int reduce_slots(int V) { return V >= 4 ? V / 4 : 1; }

template <int V>
__device__ __forceinline__ int reduce_index(int j, int lane) {
    constexpr int V1 = V >= 2 ? V / 2 : 1;
    int idx = j;
    if constexpr (V >= 2) idx += (V / 2) * ((lane >> 5) & 1);
    if constexpr (V1 >= 2) idx += (V1 / 2) * ((lane >> 4) & 1);
    return idx;
}

// True for the one lane per distinct total that should publish slot j.
template <int V>
__device__ __forceinline__ bool reduce_writer(int j, int lane) {
    constexpr int V1 = V >= 2 ? V / 2 : 1;
    bool w = (lane & 15) == j;
    if constexpr (V < 2) w = w && ((lane & 32) == 0);
    if constexpr (V1 < 2) w = w && ((lane & 16) == 0);
    return w;
}

template <int V>
__device__ __forceinline__ void wave_reduce(float (&v)[V]) {
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    if constexpr (V >= 2) {
#pragma unroll
        for (int j = 0; j < V / 2; ++j) {
            auto p = __builtin_amdgcn_permlane32_swap(fbits(v[j]), fbits(v[j + V / 2]), false, false);
            v[j] = bitsf(p[0]) + bitsf(p[1]);
        }
    } else {
        auto p = __builtin_amdgcn_permlane32_swap(fbits(v[0]), fbits(v[0]), false, false);
        v[0] = bitsf(p[0]) + bitsf(p[1]);
    }
    constexpr int V1 = V >= 2 ? V / 2 : 1;
    if constexpr (V1 >= 2) {
#pragma unroll
        for (int j = 0; j < V1 / 2; ++j) {
            auto p = __builtin_amdgcn_permlane16_swap(fbits(v[j]), fbits(v[j + V1 / 2]), false, false);
            v[j] = bitsf(p[0]) + bitsf(p[1]);
        }
    } else {
        auto p = __builtin_amdgcn_permlane16_swap(fbits(v[0]), fbits(v[0]), false, false);
        v[0] = bitsf(p[0]) + bitsf(p[1]);
    }
    constexpr int V2 = V1 >= 2 ? V1 / 2 : 1;
#pragma unroll
    for (int j = 0; j < V2; ++j) {
        v[j] += dpp<0xB1>(v[j]);    // quad_perm [1,0,3,2]
        v[j] += dpp<0x4E>(v[j]);    // quad_perm [2,3,0,1]
        v[j] += dpp<0x141>(v[j]);   // row_half_mirror
        v[j] += dpp<0x140>(v[j]);   // row_mirror
    }
}

// After wave_reduce: call f(index, total) once per value index, from the one
// lane that publishes it.  Each slot is handled by its own (predicated) call,
// so the per-lane values are never indexed dynamically.
template <int V, typename F>
__device__ __forceinline__ void for_each_reduced(const float (&v)[V], int lane, F&& f) {
    constexpr int S = reduce_slots(V);
#pragma unroll
    for (int s = 0; s < S; ++s)
        if (reduce_writer<V>(s, lane)) f(reduce_index<V>(s, lane), v[s]);
}

// Nearest bfloat16 pattern to a binary32 value, ties to even (finite values;
// values beyond the largest finite bf16 round to infinity).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = fbits(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// RMSNorm prologue of a batch-1 product (tinyinfer post, decode section: the
// normalisation folded into the projection kernel), on the token row staged in
// LDS: h[k] = bf16(x[k] g[k] / sqrt(sum_k x[k]^2 / K + eps)).  x and g are K bf16
// in natural order (K / 8 16-byte units each), already visible to the whole
// workgroup.  Only LDS is waited for: weight loads stay in flight.
//
// rms_inv_lds: 1 / sqrt(sum_k x[k]^2 / K + eps), the same value in every
// thread.  The sum of squares is fp32: per-thread partial sums, the wavefront
// tree, then the four wavefront totals in a fixed order.  Ends with a barrier.
__device__ __forceinline__ float rms_inv_lds(const u32x4* x, int K, float eps) {
    __shared__ float part[4];
    const int n = K >> 3;
    float ss[1] = {0.f};
    for (int i = threadIdx.x; i < n; i += kBlock) {
        const u32x4 v = x[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = bitsf(v[j] << 16), hi = bitsf(v[j] & 0xFFFF0000u);
            ss[0] = fmaf(lo, lo, ss[0]);
            ss[0] = fmaf(hi, hi, ss[0]);
        }
    }
    wave_reduce<1>(ss);
    if ((threadIdx.x & 63) == 0) part[wave_id()] = ss[0];
    wait_cnt<63, 0>();
    barrier_only();
    return 1.f / sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)K + eps);
}

// h for one 16-byte unit of x and the matching unit of g: x g is exact in
// fp32, the product with inv is rounded once to fp32 and once to bf16.
__device__ __forceinline__ u32x4 rms_scale_unit(const u32x4& v, const u32x4& gv, float inv) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = bitsf(v[j] << 16) * bitsf(gv[j] << 16) * inv;
        const float hi = bitsf(v[j] & 0xFFFF0000u) * bitsf(gv[j] & 0xFFFF0000u) * inv;
        o[j] = bf16_rne(lo) | (bf16_rne(hi) << 16);
    }
    return o;
}

// The whole prologue in place on the staged row (the bf16 products read it as is).
__device__ __forceinline__ void rms_norm_lds(u32x4* x, const u32x4* g, int K, float eps) {
    const float inv = rms_inv_lds(x, K, eps);
    for (int i = threadIdx.x; i < (K >> 3); i += kBlock) x[i] = rms_scale_unit(x[i], g[i], inv);
    wait_cnt<63, 0>();
    barrier_only();
}

// Matrix-core tile order.  Workgroups are dispatched round-robin over the
// eight XCDs, each with its own L2.  The workgroups that read the same W block
// (one n tile and k split, every token tile m) get consecutive slots on one
// XCD, so the block comes from HBM once and from that XCD's L2 for the other
// token tiles.  Grid: ceil(n_tiles * S / 8) * 8 * m_tiles; false for a padding
// slot (the whole workgroup leaves).
__device__ __forceinline__ bool tile_of(int b, int n_tiles, int m_tiles, int S, int& n_tile,
                                        int& ks, int& m_tile) {
    const int xcd = b & 7, loc = b >> 3;
    const int grp = (loc / m_tiles) * 8 + xcd;   // n_tile * S + ks
    m_tile = loc - (loc / m_tiles) * m_tiles;
    n_tile = grp / S;
    ks = grp - n_tile * S;
    return n_tile < n_tiles;
}
__host__ __device__ inline unsigned tile_grid(int n_tiles, int m_tiles, int S) {
    return (unsigned)(((n_tiles * S + 7) / 8) * 8 * m_tiles);
}

// Split-K workspace: a fixed region of 32-bit tile counters (zero whenever no
// kernel runs) followed by the partial tiles.  The counter region never holds
// partial data, so shapes with different tile counts can share the workspace.
constexpr int kMaxTileCounters = 1 << 16;
__host__ __device__ inline size_t ws_counter_bytes(int) { return (size_t)kMaxTileCounters * 4; }

}  // namespace lin

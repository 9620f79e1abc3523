// int4-g64 streaming product on the vector ALUs: w[n][k] = q[n][k] * s[n][k/64],
// y[m][n] = sum_k w[n][k] x[m][k], for M <= 8 tokens.  4-bit weights with one
// fp16 scale per 64 (tinyinfer post, TL;DR) cut the streamed bytes to 0.53 B
// per weight; unpacking must then cost almost nothing, since it is no longer
// hidden behind the memory traffic (llm-rs benchmark post, section 6).
//
// Mapping.  As the bf16 kernel: four wavefronts per workgroup, a wavefront owns
// R rows, each lane reads consecutive 16-byte chunks = 32 codes = half a scale
// group, so lanes 2i and 2i+1 share one scale.
//
// Unpacking without conversions (q4_unpack2): one 3-input bitwise operation
// per pair of nibbles yields two exact bf16 "codes" 24 + q that go straight
// into v_dot2_f32_bf16.  Nibble i of a dword is paired with nibble i+4, i.e.
// k = 8d+i with k = 8d+i+4, so x is re-paired the same way (one v_perm per
// pair).  The offset is removed per chunk: sum_k q x = dot(codes, x) - 24 *
// sum_k x, where sum_k x over the chunk is shared by all rows; the dot chain
// starts from -24 * sum x.  Then acc += s * chunk sum.  Per 32 weights and
// row: 24 unpack + 16 dot2 + 1 for the scale, about 1.3 vector operations per
// weight.
//
// x handling: either re-paired from cached global loads per chunk (cost shared
// by the R rows), or, with STAGE, staged once per workgroup.  Per chunk a lane
// needs 64 bytes of x for 16 bytes of weights, and those per-lane x loads
// touch four times as many cache lines as the weight loads; they cost more of
// the compute unit's load bandwidth than the weights themselves.  STAGE
// copies x into LDS with coalesced direct-to-LDS loads issued before the
// first weight loads, waits for those copies only, re-pairs x cooperatively
// into [MT][4][chunks] 16-byte words (bank-conflict-free reads) plus the
// chunk sums, and then reads x from LDS; all of this overlaps the latency of
// the first weight stage.
//
// Epilogues (EPI) as in the bf16 kernel: the residual add, or the gated
// product silu(g) u over a matrix of 2N rows (gate rows, then up rows).
// Prologue (NORM, batch 1 with x staged): the RMSNorm of x on the staged raw
// copy (rms_norm_lds, gain staged beside it), before x is re-paired.
#pragma once

#include <type_traits>

#include "kern_common.h"

namespace lin {

// 16 re-paired x dwords of one 32-k chunk: pair (x[8d+i], x[8d+i+4]) at 4d+i.
struct XChunk {
    u32x4 v[4];
    float negsum;   // -24 * sum of the 32 x values
};

__device__ __forceinline__ void pair_x(const u32x4 (&xd)[4], XChunk& out) {
    // xd[t/4][t%4] = natural dword t = (x[2t], x[2t+1]); dword d of the weights
    // covers k = 8d .. 8d+7, i.e. natural dwords 4d .. 4d+3.
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t a0 = xd[d][0], a1 = xd[d][1], a2 = xd[d][2], a3 = xd[d][3];
        out.v[d][0] = __builtin_amdgcn_perm(a2, a0, 0x05040100u);   // x0, x4
        out.v[d][1] = __builtin_amdgcn_perm(a2, a0, 0x07060302u);   // x1, x5
        out.v[d][2] = __builtin_amdgcn_perm(a3, a1, 0x05040100u);   // x2, x6
        out.v[d][3] = __builtin_amdgcn_perm(a3, a1, 0x07060302u);   // x3, x7
        s = dot2(a0, 0x3F803F80u, s);   // bf16 (1.0, 1.0)
        s = dot2(a1, 0x3F803F80u, s);
        s = dot2(a2, 0x3F803F80u, s);
        s = dot2(a3, 0x3F803F80u, s);
    }
    out.negsum = -kQ4Offset * s;
}

// One 16-byte unit of x (natural dwords d0..d3 = x[8d+0..7] of a chunk's unit
// d) re-paired as pair_x does for it, and the unit's sum of its 8 values.
__device__ __forceinline__ u32x4 pair_unit(const u32x4& a, float& s) {
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(a[2], a[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(a[2], a[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(a[3], a[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(a[3], a[1], 0x07060302u);
    s = dot2(a[0], 0x3F803F80u, 0.f);
    s = dot2(a[1], 0x3F803F80u, s);
    s = dot2(a[2], 0x3F803F80u, s);
    s = dot2(a[3], 0x3F803F80u, s);
    return o;
}

// Sum over one chunk of 32 codes times re-paired x, minus the code offset:
// 16 bitwise operations, 8 64-bit shifts and 16 dot products per 32 codes.
__device__ __forceinline__ float chunk_dot(const u32x4& wq, const XChunk& xc) {
    float acc = xc.negsum;
#pragma unroll
    for (int d = 0; d < 4; d += 2) {
        uint32_t o[8];
        q4_unpack2((uint64_t)wq[d] | ((uint64_t)wq[d + 1] << 32), o);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = dot2(o[i], xc.v[d][i], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = dot2(o[4 + i], xc.v[d + 1][i], acc);
    }
    return acc;
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// LDS layout of the staged x (16-byte units): re-paired words MT * 4 * nch,
// chunk sums MT * nch floats rounded up to whole units, then the raw copy.
__host__ __device__ inline size_t q4_stage_raw_offset(int MT, int K) {
    const size_t nch = (size_t)(K / 32);
    return (size_t)MT * 4 * nch + ((size_t)MT * nch + 3) / 4;
}
__host__ __device__ inline size_t q4_stage_bytes(int MT, int K) {
    return 16 * (q4_stage_raw_offset(MT, K) + stage_x_units(MT, K));
}

// One row block (R x 4/SPLIT rows) of the product, one per workgroup.
template <int MT, int R0, int U, int SPLIT, bool STAGE, int EPI = kEpiNone, bool NORM = false>
__device__ __forceinline__ void gemv_q4_valu_block(const KArgs& a, int64_t block) {
    static_assert(!NORM || (STAGE && MT == 1), "the prologue works on one staged token row");
    constexpr int GROUPS = 4 / SPLIT;
    constexpr int R = EPI == kEpiSwiglu ? 2 * R0 : R0;   // weight rows per wavefront
    constexpr int V = R * MT;
    constexpr int STEP = kWave * U;   // chunks per pipeline step
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = wave / SPLIT;
    const int part = wave - grp * SPLIT;
    const int M = a.M, N = a.N, K = a.K;
    const int nch = K >> 5;   // 16-byte chunks (32 codes) per row
    const int G = K >> 6;     // scale groups per row
    const uint8_t* __restrict__ Wq = (const uint8_t*)a.W;
    const uint16_t* __restrict__ S = (const uint16_t*)a.S;
    const uint16_t* __restrict__ X = (const uint16_t*)a.X;

    // STAGE: [MT][4][nch] re-paired words, [MT][nch] chunk sums (padded to
    // 16 bytes), then the raw copy of x (q4_stage_raw_offset); NORM: then the gain.
    extern __shared__ u32x4 xs[];
    float* xsum = (float*)(xs + (size_t)MT * 4 * nch);
    u32x4* xraw = xs + q4_stage_raw_offset(MT, K);
    if constexpr (STAGE) stage_x_dma(X, M, MT, K, xraw);
    if constexpr (NORM) stage_x_dma(a.G, 1, 1, K, xraw + stage_x_units(MT, K));

    const int64_t row0 = (block * GROUPS + grp) * R0;   // first output row
    const uint8_t* wb[R];
    const uint8_t* sb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t row = row0 + r % R0;
        row = row < N ? row : N - 1;   // rows past N recompute row N-1; never stored
        if (r >= R0) row += N;         // the up row of a gated product
        wb[r] = Wq + row * (int64_t)(K / 2);
        sb[r] = (const uint8_t*)(S + row * (int64_t)G);
    }
    const uint8_t* xb[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xb[m] = (const uint8_t*)(X + (size_t)(m < M ? m : 0) * K);

    const int per = (nch + SPLIT - 1) / SPLIT;
    const int cbeg = part * per;
    const int cend = min(nch, cbeg + per);

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    struct Stage {
        u32x4 w[U][R];
        uint16_t sc[U][R];
        u32x4 x[U][MT][STAGE ? 1 : 4];   // raw x of the chunk (unstaged x only)
    };
    // Every step, the last one included, loads U x 64 chunks per row; in a
    // partial last step the lanes past cend re-load chunk cend - 1 (in bounds)
    // and drop its product, so the ragged end rides the same two-stage
    // pipeline instead of a serial tail.
    auto load = [&](Stage& s, int cb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = (uint32_t)min(cb + kWave * u + lane, cend - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                s.w[u][r] = load_w16(wb[r], c * 16u);
                s.sc[u][r] = load_w2(sb[r], (c >> 1) * 2u);
            }
            if constexpr (!STAGE) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int t = 0; t < 4; ++t) s.x[u][m][t] = load_x16(xb[m], (4 * c + t) * 16u);
            }
        }
    };
    auto get_x = [&](const Stage& s, int u, int m, int c, XChunk& xc) {
        if constexpr (STAGE) {
#pragma unroll
            for (int t = 0; t < 4; ++t) xc.v[t] = xs[(m * 4 + t) * nch + c];
            xc.negsum = xsum[m * nch + c];
        } else {
            pair_x(s.x[u][m], xc);
        }
    };
    auto compute = [&](const Stage& s, int cb, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + kWave * u + lane;
            const int cc = min(c, cend - 1);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                XChunk xc;
                get_x(s, u, m, cc, xc);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    // lanes past cend unpack zero codes in the partial step (the
                    // result is dropped): the two step forms then differ, so the
                    // compiler does not hoist a whole stage's unpacking above
                    // the step branch and keep it live
                    const u32x4 wq = (MASK && c >= cend) ? u32x4{0u, 0u, 0u, 0u} : s.w[u][r];
                    const float v = fmaf(half_to_float(s.sc[u][r]), chunk_dot(wq, xc),
                                         acc[r * MT + m]);
                    if constexpr (MASK)
                        acc[r * MT + m] = c < cend ? v : acc[r * MT + m];
                    else
                        acc[r * MT + m] = v;
                }
            }
        }
    };
    auto step = [&](const Stage& s, int cb) {
        if (cb + STEP > cend)
            compute(s, cb, std::true_type{});
        else
            compute(s, cb, std::false_type{});
    };

    // two register stages in flight (unrolled by two: no copies)
    const int nsteps = cend > cbeg ? (cend - cbeg + STEP - 1) / STEP : 0;
    int cb = cbeg;
    Stage s0, s1;
    if (nsteps > 0) load(s0, cb);
    bool s1_early = false;
    if constexpr (STAGE) {
        // Both weight stages (2 U R loads each: codes and scales) are issued
        // before waiting for the x copies, so that they stream while x lands,
        // is normalised and re-paired.  The copies were issued first and loads
        // complete in order: waiting down to the weight loads leaves them in
        // flight.  The barrier makes every wavefront's copies visible.
        if (nsteps > 1) {
            load(s1, cb + STEP);
            s1_early = true;
            wait_cnt<4 * U * R, 15>();
        } else if (nsteps > 0) {
            wait_cnt<2 * U * R, 15>();
        } else {
            wait_cnt<0, 15>();
        }
        barrier_only();
        // One thread per 16-byte unit: re-pair it (with NORM, normalise it
        // first) and sum its values; the four units of a chunk sit in the
        // four lanes of a quad (K / 8 is a multiple of 4), which add their
        // sums with two DPP steps.
        float inv = 1.f;
        if constexpr (NORM) inv = rms_inv_lds(xraw, K, a.eps);
        const u32x4* graw = xraw + stage_x_units(MT, K);
        const int upr = K >> 3;   // 16-byte units per token row
        for (int u = threadIdx.x; u < MT * upr; u += kBlock) {
            const int m = u / upr;
            const int j = u - m * upr;
            const int c = j >> 2, d = j & 3;
            u32x4 v = xraw[u];
            if constexpr (NORM) v = rms_scale_unit(v, graw[j], inv);
            float sum;
            const u32x4 p = pair_unit(v, sum);
            sum += dpp<0xB1>(sum);   // quad_perm [1,0,3,2]
            sum += dpp<0x4E>(sum);   // quad_perm [2,3,0,1]
            xs[(m * 4 + d) * nch + c] = p;
            if (d == 0) xsum[m * nch + c] = -kQ4Offset * sum;
        }
        wait_cnt<63, 0>();   // LDS writes done, weight loads still in flight
        barrier_only();
    }
    if (nsteps > 0) {
        for (int it = 0;;) {
            if (it + 1 < nsteps && !(it == 0 && s1_early)) load(s1, cb + STEP);
            step(s0, cb);
            cb += STEP;
            if (++it >= nsteps) break;
            if (it + 1 < nsteps) load(s0, cb + STEP);
            step(s1, cb);
            cb += STEP;
            if (++it >= nsteps) break;
        }
    }

    wave_reduce<V>(acc);
    if constexpr (EPI == kEpiSwiglu) {
        // gate and up totals land in different lanes: meet in LDS
        __shared__ float red[4][V];
        for_each_reduced<V>(acc, lane, [&](int idx, float val) { red[wave][idx] = val; });
        __syncthreads();
        if (part == 0) {
            for (int j = lane; j < R0 * MT; j += kWave) {
                const int r = j / MT, m = j - (j / MT) * MT;
                float g = red[wave][j], u = red[wave][R0 * MT + j];
#pragma unroll
                for (int p = 1; p < SPLIT; ++p) {
                    g += red[wave + p][j];
                    u += red[wave + p][R0 * MT + j];
                }
                if (m < M && row0 + r < N) a.Y[(int64_t)m * N + row0 + r] = silu_mul(g, u);
            }
        }
    } else if constexpr (SPLIT == 1) {
        for_each_reduced<V>(acc, lane, [&](int idx, float val) {
            const int r = idx / MT, m = idx - (idx / MT) * MT;
            const int64_t o = (int64_t)m * N + row0 + r;
            if (m < M && row0 + r < N) a.Y[o] = EPI == kEpiAdd ? val + a.R[o] : val;
        });
    } else {
        __shared__ float red[4][V];
        for_each_reduced<V>(acc, lane, [&](int idx, float val) { red[wave][idx] = val; });
        __syncthreads();
        if (part == 0) {
            for_each_reduced<V>(acc, lane, [&](int idx, float) {
                const int r = idx / MT, m = idx - (idx / MT) * MT;
                float s = red[wave][idx];
#pragma unroll
                for (int p = 1; p < SPLIT; ++p) s += red[wave + p][idx];
                const int64_t o = (int64_t)m * N + row0 + r;
                if (m < M && row0 + r < N) a.Y[o] = EPI == kEpiAdd ? s + a.R[o] : s;
            });
        }
    }
}

}  // namespace lin

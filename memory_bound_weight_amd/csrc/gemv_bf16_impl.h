// bf16 streaming product on the vector ALUs: y[m][n] = sum_k W[n][k] x[m][k]
// for a few tokens (M <= 32).  The weights are streamed from HBM exactly once
// (llm-rs benchmark post, section 2: decode is weight streaming); the tokens of
// a batch share each loaded weight (section 3 of the same post).
//
// Mapping.  A workgroup is four wavefronts.  A wavefront owns R consecutive
// rows; its 64 lanes read consecutive 16-byte chunks of each row (eight bf16),
// so one wavefront load instruction covers 1 KiB of a row, and a lane keeps
// U x R independent loads in flight (tinyinfer post, "v0.2": several rows per
// warp keep more requests in flight).  The loop is software-pipelined: the
// loads of step i+1 are issued before the products of step i.  With SPLIT > 1,
// SPLIT wavefronts share the same rows, each taking a contiguous part of K, and
// combine through LDS; this fills the chip when N is small.  x is read through
// the cache hierarchy, or, when STAGE is set, copied into LDS once per
// workgroup with coalesced direct-to-LDS loads issued before the first weight
// loads (only those copies are waited for, so the copy overlaps the latency
// of the first weight stage).
// Products use v_dot2_f32_bf16 (two exact bf16 products per instruction, fp32
// sums); each lane sums K/512 chunks, then a permlane/DPP tree sums the lanes.
//
// Epilogues (EPI, yalm post, GPU matmul section: fold the next elementwise
// step into the product that feeds it): kEpiAdd writes y = W x + r (the
// residual add, r may be y itself); kEpiSwiglu reads a weight matrix of 2N
// rows (gate rows, then up rows, as concatenated at load), gives each
// wavefront R0 gate rows and the R0 matching up rows, and writes
// y[n] = silu(g_n) u_n, so the gated activation never makes a round trip.
//
// Prologue (NORM, batch 1 with x staged): the RMSNorm of x is formed on the
// staged copy (rms_norm_lds) before the first product; its gain vector is
// staged next to x by the same direct-to-LDS copies, so the whole prologue
// overlaps the latency of the first weight stage, like the staging itself.
#pragma once

#include <type_traits>

#include "kern_common.h"

namespace lin {

// One row block (R x 4/SPLIT rows) of the product, one per workgroup.
template <int MT, int R0, int U, int SPLIT, bool STAGE, int EPI = kEpiNone, bool NORM = false>
__device__ __forceinline__ void gemv_bf16_valu_block(const KArgs& a, int64_t block) {
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
    const int nch = K >> 3;   // 16-byte chunks per row
    const uint16_t* __restrict__ W = (const uint16_t*)a.W;
    const uint16_t* __restrict__ X = (const uint16_t*)a.X;

    extern __shared__ u32x4 xs[];   // STAGE: [MT][nch] chunks of x; NORM: then the gain
    if constexpr (STAGE) stage_x_dma(X, M, MT, K, xs);
    if constexpr (NORM) stage_x_dma(a.G, 1, 1, K, xs + stage_x_units(MT, K));

    const int64_t row0 = (block * GROUPS + grp) * R0;   // first output row
    const uint8_t* wb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t row = row0 + r % R0;
        row = row < N ? row : N - 1;   // rows past N recompute row N-1; never stored
        if (r >= R0) row += N;         // the up row of a gated product
        wb[r] = (const uint8_t*)(W + row * (int64_t)K);
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
        u32x4 x[U][MT];
    };
    // Every step, the last one included, loads U x 64 chunks per row; in a
    // partial last step the lanes past cend re-load chunk cend - 1 (in bounds)
    // and drop its product, so the ragged end rides the same two-stage
    // pipeline instead of a serial tail.
    auto load = [&](Stage& s, int cb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(cb + kWave * u + lane, cend - 1);
            const uint32_t off = (uint32_t)c * 16u;
#pragma unroll
            for (int r = 0; r < R; ++r) s.w[u][r] = load_w16(wb[r], off);
            if constexpr (!STAGE) {
#pragma unroll
                for (int m = 0; m < MT; ++m) s.x[u][m] = load_x16(xb[m], off);
            }
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
                const u32x4 xv = STAGE ? xs[m * nch + cc] : s.x[u][m];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if constexpr (MASK) {
                        float t = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) t = dot2(s.w[u][r][j], xv[j], t);
                        acc[r * MT + m] += c < cend ? t : 0.f;
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[r * MT + m] = dot2(s.w[u][r][j], xv[j], acc[r * MT + m]);
                    }
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
        // Both weight stages are issued before waiting for the x copies, so
        // that they stream while x lands (and is normalised).  The copies were
        // issued first and loads complete in order: waiting down to the weight
        // loads leaves them in flight.  The barrier makes every wavefront's
        // copies visible.
        if (nsteps > 1) {
            load(s1, cb + STEP);
            s1_early = true;
            wait_cnt<2 * U * R, 15>();
        } else if (nsteps > 0) {
            wait_cnt<U * R, 15>();
        } else {
            wait_cnt<0, 15>();
        }
        barrier_only();
        if constexpr (NORM) rms_norm_lds(xs, xs + stage_x_units(MT, K), K, a.eps);
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
        __syncthreads();
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
        __syncthreads();
    }
}

}  // namespace lin

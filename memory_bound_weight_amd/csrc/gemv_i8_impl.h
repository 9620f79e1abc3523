// INT8 streaming product on the vector ALUs, one fp32 scale per output
// channel: y[m][n] = s[n] * sum_k q[n][k] x[m][k] for M <= 8 tokens (TileInfer.jl
// post, "Pushing further with cheating: INT8 quantization": the INT8 values
// are multiplied in and the channel's scale is applied once at the end).  One
// byte per weight halves the bf16 stream.
//
// Mapping.  As the bf16 kernel: four wavefronts per workgroup, a wavefront
// owns R rows, each lane reads consecutive 16-byte chunks (16 weights) of a
// row with a two-stage register pipeline, SPLIT wavefronts may share rows
// along K, x comes through the caches or is staged in LDS once per workgroup.
//
// Conversion.  Each code byte becomes an fp32 with one v_cvt_f32_i32 that
// reads the byte in place, sign-extended (a sub-dword operand select), so a
// weight costs one conversion and one fp32 fma with x, whose bf16 values
// become fp32 by a shift (shared by the R rows).  Every product q x is exact
// in fp32 and there is no offset to remove, so the rounding of the sums is
// relative to sum_k |q x|.  The wavefront then reduces as usual and one lane
// per output multiplies by the row's scale.
//
// Epilogues and prologue (batch 1) as in the bf16 kernel: EPI adds the
// residual, or forms silu(s_g g) (s_u u) over the gate|up rows (each row's
// own scale applied before the gate); NORM normalises the staged x in place
// (RMSNorm, gain staged beside x) before the first product.
#pragma once

#include <type_traits>

#include "kern_common.h"

namespace lin {

template <int MT, int R0, int U, int SPLIT, bool STAGE, int EPI = kEpiNone, bool NORM = false>
__device__ __forceinline__ void gemv_i8_valu_block(const KArgs& a, int64_t block) {
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
    const int nch = K >> 4;   // 16-byte chunks (16 weights) per row
    const int xun = K >> 3;   // 16-byte units of x per token row
    const int8_t* __restrict__ W = (const int8_t*)a.W;
    const float* __restrict__ S = (const float*)a.S;
    const uint16_t* __restrict__ X = (const uint16_t*)a.X;

    extern __shared__ u32x4 xs[];   // STAGE: [MT][K/8] units of x; NORM: then the gain
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
        u32x4 x[U][MT][STAGE ? 1 : 2];   // the chunk's 16 x values (unstaged x only)
    };
    // As in the bf16 kernel, a partial last step re-loads chunk cend - 1 in
    // the lanes past cend and drops its products.
    auto load = [&](Stage& s, int cb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(cb + kWave * u + lane, cend - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) s.w[u][r] = load_w16(wb[r], (uint32_t)c * 16u);
            if constexpr (!STAGE) {
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    s.x[u][m][0] = load_x16(xb[m], (uint32_t)c * 32u);
                    s.x[u][m][1] = load_x16(xb[m], (uint32_t)c * 32u + 16u);
                }
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
                u32x4 x0, x1;
                if constexpr (STAGE) {
                    x0 = xs[m * xun + 2 * cc];
                    x1 = xs[m * xun + 2 * cc + 1];
                } else {
                    x0 = s.x[u][m][0];
                    x1 = s.x[u][m][1];
                }
                float xf[16];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t d = i < 4 ? x0[i] : x1[i - 4];
                    xf[2 * i] = bitsf(d << 16);
                    xf[2 * i + 1] = bitsf(d & 0xFFFF0000u);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float p = MASK ? 0.f : acc[r * MT + m];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // In the partial last step the lanes past cend convert
                        // zero codes: their results differ from the full steps',
                        // so the compiler cannot hoist a stage's conversions
                        // above the step branch (which would keep them all live).
                        const uint32_t wj = (MASK && c >= cend) ? 0u : s.w[u][r][j];
#pragma unroll
                        for (int e = 0; e < 4; ++e)   // the signed byte e of wj, exactly
                            p = fmaf((float)(int8_t)(wj >> (8 * e)), xf[4 * j + e], p);
                    }
                    if constexpr (MASK)
                        acc[r * MT + m] += c < cend ? p : 0.f;
                    else
                        acc[r * MT + m] = p;
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

    const int nsteps = cend > cbeg ? (cend - cbeg + STEP - 1) / STEP : 0;
    int cb = cbeg;
    Stage s0, s1;
    if (nsteps > 0) load(s0, cb);
    bool s1_early = false;
    if constexpr (STAGE) {
        // both weight stages stream while the x copies land (see the bf16 kernel)
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
    // y = scale * total (no scale read when K == 0), then the epilogue
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
                if (m < M && row0 + r < N) {
                    const float sg = K > 0 ? S[row0 + r] : 0.f;
                    const float su = K > 0 ? S[N + row0 + r] : 0.f;
                    a.Y[(int64_t)m * N + row0 + r] = silu_mul(sg * g, su * u);
                }
            }
        }
        __syncthreads();
    } else if constexpr (SPLIT == 1) {
        for_each_reduced<V>(acc, lane, [&](int idx, float val) {
            const int r = idx / MT, m = idx - (idx / MT) * MT;
            const int64_t o = (int64_t)m * N + row0 + r;
            if (m < M && row0 + r < N) {
                const float v = K > 0 ? S[row0 + r] * val : 0.f;
                a.Y[o] = EPI == kEpiAdd ? v + a.R[o] : v;
            }
        });
    } else {
        __shared__ float red[4][V];
        for_each_reduced<V>(acc, lane, [&](int idx, float val) { red[wave][idx] = val; });
        __syncthreads();
        if (part == 0) {
            for_each_reduced<V>(acc, lane, [&](int idx, float) {
                const int r = idx / MT, m = idx - (idx / MT) * MT;
                float t = red[wave][idx];
#pragma unroll
                for (int p = 1; p < SPLIT; ++p) t += red[wave + p][idx];
                const int64_t o = (int64_t)m * N + row0 + r;
                if (m < M && row0 + r < N) {
                    const float v = K > 0 ? S[row0 + r] * t : 0.f;
                    a.Y[o] = EPI == kEpiAdd ? v + a.R[o] : v;
                }
            });
        }
        __syncthreads();
    }
}

}  // namespace lin

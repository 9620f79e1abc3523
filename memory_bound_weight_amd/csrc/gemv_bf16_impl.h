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
// the cache hierarchy, or staged in LDS once per workgroup when STAGE is set.
// Products use v_dot2_f32_bf16 (two exact bf16 products per instruction, fp32
// sums); each lane sums K/512 chunks, then a permlane/DPP tree sums the lanes.
#pragma once

#include "kern_common.h"

namespace lin {

// One row block (R x 4/SPLIT rows) of the product, one per workgroup.
template <int MT, int R, int U, int SPLIT, bool STAGE>
__device__ __forceinline__ void gemv_bf16_valu_block(const KArgs& a, int64_t block) {
    constexpr int GROUPS = 4 / SPLIT;
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

    extern __shared__ u32x4 xs[];   // STAGE: [MT][nch] chunks of x
    if constexpr (STAGE) {
        for (int i = threadIdx.x; i < MT * nch; i += kBlock) {
            const int m = i / nch;
            const int c = i - m * nch;
            const int mm = m < M ? m : 0;
            xs[i] = load_x16((const uint8_t*)(X + (size_t)mm * K), (uint32_t)c * 16u);
        }
        __syncthreads();
    }

    const int64_t row0 = (block * GROUPS + grp) * R;
    const uint8_t* wb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t row = row0 + r;
        row = row < N ? row : N - 1;   // rows past N recompute row N-1; never stored
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
    auto load = [&](Stage& s, int cb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = (uint32_t)(cb + kWave * u + lane) * 16u;
#pragma unroll
            for (int r = 0; r < R; ++r) s.w[u][r] = load_w16(wb[r], off);
            if constexpr (!STAGE) {
#pragma unroll
                for (int m = 0; m < MT; ++m) s.x[u][m] = load_x16(xb[m], off);
            }
        }
    };
    auto compute = [&](const Stage& s, int cb) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const u32x4 xv = STAGE ? xs[m * nch + cb + kWave * u + lane] : s.x[u][m];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[r * MT + m] = dot2(s.w[u][r][j], xv[j], acc[r * MT + m]);
            }
    };

    // full steps, two register stages in flight (unrolled by two: no copies)
    const int nfull = (cend - cbeg) / STEP;
    int cb = cbeg;
    if (nfull > 0) {
        Stage s0, s1;
        load(s0, cb);
        for (int it = 0;;) {
            if (it + 1 < nfull) load(s1, cb + STEP);
            compute(s0, cb);
            cb += STEP;
            if (++it >= nfull) break;
            if (it + 1 < nfull) load(s0, cb + STEP);
            compute(s1, cb);
            cb += STEP;
            if (++it >= nfull) break;
        }
    }
    for (; cb < cend; cb += kWave) {   // ragged tail: one chunk per lane at most
        const int c = cb + lane;
        if (c < cend) {
            const uint32_t off = (uint32_t)c * 16u;
            u32x4 w[R];
#pragma unroll
            for (int r = 0; r < R; ++r) w[r] = load_w16(wb[r], off);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const u32x4 xv = STAGE ? xs[m * nch + c] : load_x16(xb[m], off);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[r * MT + m] = dot2(w[r][j], xv[j], acc[r * MT + m]);
            }
        }
    }

    wave_reduce<V>(acc);
    if constexpr (SPLIT == 1) {
        for_each_reduced<V>(acc, lane, [&](int idx, float val) {
            const int r = idx / MT, m = idx - (idx / MT) * MT;
            if (m < M && row0 + r < N) a.Y[(int64_t)m * N + row0 + r] = val;
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
                if (m < M && row0 + r < N) a.Y[(int64_t)m * N + row0 + r] = s;
            });
        }
        __syncthreads();
    }
}

}  // namespace lin

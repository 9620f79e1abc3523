// int4-g64 product on the vector ALUs over the tiled layout of lin_q4g64_tile,
// for one or two tokens: the small-M path of lin_gemm_skinny_q4g64.  With
// one 16-token matrix-core tile per M <= 16 and few row tiles on small
// matrices, the matrix-core kernel needs split-K, whose reduction costs
// several microseconds; this kernel streams the same tiled bytes with no
// cross-workgroup step.
//
// Mapping.  A wavefront owns R row tiles (16 rows each).  Per 128-k block, one
// lane-linear 16-byte load per row tile gives lane l the codes of row l mod 16
// for the four k-slices k0 = 128 j + 32 t + 8 (l / 16), t < 4, already in
// natural bf16 pair order (see the tiled layout); x of those slices comes
// through the caches (four 16-byte loads per token, shared by the R tiles).
// Unpacking is the GEMV's (q4_unpack2): exact bf16 codes 24 + q.  The offset
// is removed per scale group: the lane's sum of x over the group's two slices
// (shared by all rows of the wavefront) times -24 seeds the dot chain of each
// row.  The four lanes of a row (l, l + 16, l + 32,
// l + 48) are summed with permlane32/16 swaps; SPLIT wavefronts of a
// workgroup take parts of K and combine through LDS.
#pragma once

#include <type_traits>

#include "kern_common.h"

namespace lin {

template <int MT, int R, int U, int SPLIT>
__device__ __forceinline__ void gemv_q4t_valu_block(const KArgs& a, int64_t block) {
    constexpr int GROUPS = 4 / SPLIT;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    const int wave = wave_id();
    const int grp = wave / SPLIT;
    const int part = wave - grp * SPLIT;
    const int M = a.M, N = a.N, K = a.K;
    const int N16 = (N + 15) >> 4;
    const int KBn = (K + 127) >> 7;
    const uint8_t* __restrict__ Wt = (const uint8_t*)a.W;
    const uint8_t* __restrict__ St = (const uint8_t*)a.S;
    const uint8_t* __restrict__ X = (const uint8_t*)a.X;

    const int64_t tile0 = (block * GROUPS + grp) * R;   // first row tile of this wavefront
    const uint8_t* wb[R];
    int tr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t T = tile0 + r;
        T = T < N16 ? T : N16 - 1;   // tiles past the end re-read the last; never stored
        tr[r] = (int)T;
        wb[r] = Wt + T * KBn * 1024 + 16 * lane;
    }
    const uint8_t* xb[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xb[m] = X + (size_t)(m < M ? m : 0) * K * 2;

    const int per = (KBn + SPLIT - 1) / SPLIT;
    const int jbeg = part * per;
    const int jend = min(KBn, jbeg + per);

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    // A stage is U consecutive 128-k blocks; blocks past jend re-load the last
    // block (in bounds) and are dropped.
    struct Unit {
        u32x4 w[R];
        uint32_t s[R];
        u32x4 x[MT][4];
    };
    struct Stage {
        Unit u[U];
    };
    auto load_unit = [&](Unit& st, int j) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            st.w[r] = load_w16(wb[r], (uint32_t)j * 1024u);
            st.s[r] = __builtin_nontemporal_load(
                (const uint32_t*)(St + ((int64_t)j * N16 + tr[r]) * 64 + 4 * l16));
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 128 * j + 32 * t + 8 * lg;
                // k >= K only in the last block of a K that is not a multiple of 128
                st.x[m][t] = load_x16(xb[m], (uint32_t)(k < K ? k : 0) * 2u);
                if (k >= K) st.x[m][t] = u32x4{0u, 0u, 0u, 0u};
            }
    };
    auto load = [&](Stage& st, int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) load_unit(st.u[u], min(j + u, jend - 1));
    };
    auto compute_unit = [&](const Unit& st) {
        // -24 x the lane's sum of x over each scale group (t = 0, 1 and t = 2, 3)
        float neg[MT][2];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float s = 0.f;
#pragma unroll
                for (int t = 2 * h; t < 2 * h + 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s = dot2(st.x[m][t][i], 0x3F803F80u, s);
                neg[m][h] = -kQ4Offset * s;
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t c[4][4];   // bf16 code pairs of slice t: natural k pairs i
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                uint32_t o[8];
                q4_unpack2((uint64_t)st.w[r][2 * p] | ((uint64_t)st.w[r][2 * p + 1] << 32), o);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c[2 * p][i] = o[i];
                    c[2 * p + 1][i] = o[4 + i];
                }
            }
            const float s0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(st.s[r] & 0xFFFFu));
            const float s1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(st.s[r] >> 16));
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float d = neg[m][h];
#pragma unroll
                    for (int t = 2 * h; t < 2 * h + 2; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) d = dot2(c[t][i], st.x[m][t][i], d);
                    acc[r][m] = fmaf(h ? s1 : s0, d, acc[r][m]);
                }
            }
        }
    };
    auto compute = [&](const Stage& st, int j) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j + u < jend) compute_unit(st.u[u]);
    };

    // two register stages of U blocks in flight (unrolled by two: no copies)
    Stage s0, s1;
    int j = jbeg;
    if (j < jend) load(s0, j);
    while (j < jend) {
        if (j + U < jend) load(s1, j + U);
        compute(s0, j);
        j += U;
        if (j >= jend) break;
        if (j + U < jend) load(s0, j + U);
        compute(s1, j);
        j += U;
    }

    // sum the four lanes of each row: l, l ^ 32, then l, l ^ 16
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            auto p = __builtin_amdgcn_permlane32_swap(fbits(acc[r][m]), fbits(acc[r][m]), false, false);
            float v = bitsf(p[0]) + bitsf(p[1]);
            auto q = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
            acc[r][m] = bitsf(q[0]) + bitsf(q[1]);
        }
    if constexpr (SPLIT == 1) {
        if (lg == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t n = (tile0 + r) * 16 + l16;
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M && n < N) a.Y[(int64_t)m * N + n] = acc[r][m];
            }
        }
    } else {
        __shared__ float red[4][R][MT][16];
        if (lg == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) red[wave][r][m][l16] = acc[r][m];
        }
        __syncthreads();
        if (part == 0 && lg == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t n = (tile0 + r) * 16 + l16;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float t = red[wave][r][m][l16];
#pragma unroll
                    for (int p = 1; p < SPLIT; ++p) t += red[wave + p][r][m][l16];
                    if (m < M && n < N) a.Y[(int64_t)m * N + n] = t;
                }
            }
        }
    }
}

}  // namespace lin

// Matrix-core path of the batched-token product Y = X . W^T (bf16 in, fp32
// accumulate), for token counts where the product is a real dense
// contraction.  Batching M tokens raises the work per weight byte to about M
// FLOP (llm-rs benchmark post, section 3); past a few tens of tokens the vector
// ALUs can no longer keep up with HBM, so the multiply moves to MFMA.  The
// recipe follows section 5 of the same post (tiling for reuse, matrix
// instructions, pipelining, bank-conflict-free layouts), re-derived for CDNA4.
//
// Instruction: v_mfma_f32_16x16x32_bf16.  In both operands lane l holds eight
// consecutive k of row (l mod 16), lane group l/16 selecting which eight; the
// 16x16 fp32 result gives lane l column (l mod 16), rows 4(l/16) .. 4(l/16)+3.
//
// Mapping.  A workgroup is four wavefronts and owns BN = 64 NF rows of W and
// TM tokens.  Wavefront w owns NF fragments of 16 W rows.  W is the streamed
// operand: each lane loads its B fragment straight from HBM (16 bytes; the 64
// lanes cover 16 rows x 64 contiguous bytes), with the next k-block's
// fragments prefetched into registers while the current block is multiplied;
// every W byte is read once per workgroup and used against all TM tokens.
// X, re-read by every workgroup, goes through LDS: a TM x 64 tile per k-block,
// double-buffered, with 16-byte chunk c of token row m stored at slot
// c ^ (m mod 8) (XOR swizzle, no padding) so the A-fragment reads spread over
// the banks.  Each A fragment read from LDS is reused for the NF W fragments.
//
// Tile order.  Workgroups are dispatched round-robin over the eight XCDs, each
// with its own L2.  When M needs several token tiles, the tiles of one W block
// are given consecutive slots on the same XCD, so the W block comes from HBM
// once and from that XCD's L2 for the other token tiles.
#include "registry.h"

namespace lin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;   // k per block: two MFMA steps of 32

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int NF, int TM>
__global__ __launch_bounds__(kBlock) void gemm_mfma_kernel(KArgs a) {
    constexpr int BN = 64 * NF;
    constexpr int MT = TM / 16;                  // 16-token sub-tiles
    constexpr int XCH = TM * (kBK / 8) / kBlock;  // 16-byte X chunks per thread per block
    static_assert(XCH >= 1, "TM too small");
    const int M = a.M, N = a.N, K = a.K;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int l16 = lane & 15, lg = lane >> 4;

    // XCD-aware tile order (see above)
    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    const int b = blockIdx.x;
    const int xcd = b & 7, loc = b >> 3;
    const int n_tile = (loc / m_tiles) * 8 + xcd;
    const int m_tile = loc - (loc / m_tiles) * m_tiles;
    if (n_tile >= n_tiles) return;   // padding slot: whole workgroup leaves together
    const int n0 = n_tile * BN + wave * 16 * NF;
    const int m0 = m_tile * TM;

    __shared__ u32x4 xt[2][TM * (kBK / 8)];   // two X tiles, 16-byte chunks, swizzled

    const uint16_t* __restrict__ W = (const uint16_t*)a.W;
    const uint16_t* __restrict__ X = (const uint16_t*)a.X;
    const uint8_t* wrow[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        int n = n0 + f * 16 + l16;
        n = n < N ? n : N - 1;   // rows past N are computed, never stored
        wrow[f] = (const uint8_t*)(W + (int64_t)n * K);
    }

    // X chunks this thread stages: chunk q = threadIdx.x + 256 i -> row q/8, chunk q%8
    auto load_x = [&](u32x4 (&xr)[XCH], int kb) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int q = threadIdx.x + kBlock * i;
            const int m = q >> 3, c = q & 7;
            const int gm = m0 + m;
            const int k = kb * kBK + c * 8;   // K % 8 == 0: a chunk is wholly in or out
            xr[i] = (gm < M && k < K) ? load_x16((const uint8_t*)(X + (int64_t)gm * K), (uint32_t)k * 2u)
                                      : u32x4{0, 0, 0, 0};
        }
    };
    auto store_x = [&](const u32x4 (&xr)[XCH], int buf) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int q = threadIdx.x + kBlock * i;
            const int m = q >> 3, c = q & 7;
            xt[buf][m * 8 + (c ^ (m & 7))] = xr[i];
        }
    };
    auto load_w = [&](u32x4 (&wr)[NF][2], int kb) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int s = 0; s < 2; ++s)
            {
                const int k = kb * kBK + s * 32 + lg * 8;
                wr[f][s] = k < K ? load_w16(wrow[f], (uint32_t)k * 2u) : u32x4{0, 0, 0, 0};
            }
    };

    f32x4 acc[NF][MT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const u32x4 (&wr)[NF][2], int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = t * 16 + l16;
                const int c = s * 4 + lg;
                const u32x4 av = xt[buf][m * 8 + (c ^ (m & 7))];
#pragma unroll
                for (int f = 0; f < NF; ++f) acc[f][t] = mfma16(av, wr[f][s], acc[f][t]);
            }
    };

    const int nkb = (K + kBK - 1) / kBK;   // a partial last block is zero-filled
    u32x4 w0[NF][2], w1[NF][2];
    u32x4 xr[XCH];
    load_w(w0, 0);
    load_x(xr, 0);
    store_x(xr, 0);
    __syncthreads();
    // k-blocks, two register stages of W (unrolled by two: no copies)
    for (int kb = 0;;) {
        if (kb + 1 < nkb) {
            load_w(w1, kb + 1);
            load_x(xr, kb + 1);
        }
        compute(w0, kb & 1);
        if (kb + 1 < nkb) store_x(xr, (kb + 1) & 1);
        __syncthreads();
        if (++kb >= nkb) break;
        if (kb + 1 < nkb) {
            load_w(w0, kb + 1);
            load_x(xr, kb + 1);
        }
        compute(w1, kb & 1);
        if (kb + 1 < nkb) store_x(xr, (kb + 1) & 1);
        __syncthreads();
        if (++kb >= nkb) break;
    }

    // epilogue: lane holds rows 4*lg + r of each 16-token sub-tile, column l16
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
}

template <int NF, int TM>
static bool geom_mfma(const Variant&, int M, int N, int K, dim3* grid, size_t* lds) {
    if (K <= 0) return false;
    constexpr int BN = 64 * NF;
    const int m_tiles = (M + TM - 1) / TM;
    if (TM > 16 && M <= TM / 2) return false;    // a smaller token tile fits
    const int n_tiles = (N + BN - 1) / BN;
    const int n_pad = (n_tiles + 7) / 8 * 8;
    *grid = dim3((unsigned)(n_pad * m_tiles));
    *lds = 0;
    return true;
}

template <int NF, int TM>
static void add(std::vector<Variant>& out) {
    Variant v{};
    v.kind = LIN_KIND_SKINNY_BF16;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = 64 * NF;
    v.cfg.unroll = 1;
    v.cfg.split = 1;
    v.cfg.stage_x = 1;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = 16;
    v.func = (const void*)&gemm_mfma_kernel<NF, TM>;
    v.geometry = &geom_mfma<NF, TM>;
    out.push_back(v);
}

void register_gemm_mfma(std::vector<Variant>& out) {
    add<1, 32>(out);
    add<1, 64>(out);
    add<2, 64>(out);
    add<4, 64>(out);
    add<1, 128>(out);
    add<2, 128>(out);
    add<1, 256>(out);
    add<2, 256>(out);
}

}  // namespace lin

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
// lanes cover 16 rows x 64 contiguous bytes); a ring of D register stages
// keeps D k-blocks of W and X loads in flight per workgroup (one block of work
// is far too short to cover HBM latency); every W byte is read once per
// workgroup and used against all TM tokens.
// X, re-read by every workgroup, goes through LDS: a TM x 64 tile per k-block,
// double-buffered, with 16-byte chunk c of token row m stored at slot
// c ^ (m mod 8) (XOR swizzle, no padding) so the A-fragment reads spread over
// the banks.  Each A fragment read from LDS is reused for the NF W fragments.
//
// Tile order.  Workgroups are dispatched round-robin over the eight XCDs, each
// with its own L2.  When M needs several token tiles, the tiles of one W block
// are given consecutive slots on the same XCD, so the W block comes from HBM
// once and from that XCD's L2 for the other token tiles.
//
// Split-K.  A small N x M leaves too few output tiles to keep 256 CUs streaming
// (each workgroup walks K serially), so SPLITS workgroups share a tile, each
// taking a contiguous range of k-blocks.  Each writes its partial tile to the
// workspace with coherent (agent-scope) stores, waits for them to complete and
// bumps the tile's counter.  The workgroup that sees the last count adds the
// SPLITS partials in split order
// 0, 1, ... (so the result does not depend on which one finishes last), writes
// Y and resets the counter to zero for the next call.  No workgroup ever waits
// for another.
#include "mfma_common.h"
#include "registry.h"

namespace lin {

constexpr int kBK = 64;   // k per block: two MFMA steps of 32

template <int NF, int TM, int D>
__global__ __launch_bounds__(kBlock) void gemm_mfma_kernel(KArgs a) {
    constexpr int BN = 64 * NF;
    constexpr int MT = TM / 16;                  // 16-token sub-tiles
    constexpr int XCH = TM * (kBK / 8) / kBlock;  // 16-byte X chunks per thread per block
    static_assert(XCH >= 1, "TM too small");
    const int M = a.M, N = a.N, K = a.K;
    const int S = a.splits;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int l16 = lane & 15, lg = lane >> 4;

    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    int n_tile, m_tile, ks;
    if (!tile_of(blockIdx.x, n_tiles, m_tiles, S, n_tile, ks, m_tile))
        return;   // padding slot: the whole workgroup leaves together
    const int n0 = n_tile * BN + wave * 16 * NF;
    const int m0 = m_tile * TM;
    const int nkb_all = (K + kBK - 1) / kBK;   // a partial last block is zero-filled
    const int bps = (nkb_all + S - 1) / S;     // k-blocks per split
    const int kb0 = ks * bps;
    const int kb1 = min(nkb_all, kb0 + bps);

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
            for (int s = 0; s < 2; ++s) {
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

    // D-stage prefetch ring: the loads of block kb + D are issued as soon as
    // block kb has been consumed, so D blocks of W (and of X) are in flight per
    // workgroup.  The ring is unrolled by D so every stage index is static.
    struct Stage {
        u32x4 w[NF][2];
        u32x4 x[XCH];
    };
    Stage st[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (kb0 + d < kb1) {
            load_w(st[d].w, kb0 + d);
            load_x(st[d].x, kb0 + d);
        }
    for (int base = kb0; base < kb1; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int kb = base + d;
            if (kb >= kb1) break;
            const int buf = (kb - kb0) & 1;
            store_x(st[d].x, buf);
            // X tile complete (LDS writes done; later stages' loads stay in
            // flight, which __syncthreads would drain); the buffer written
            // next time is idle.
            wait_cnt<63, 0>();
            barrier_only();
            compute(st[d].w, buf);
            if (kb + D < kb1) {
                load_w(st[d].w, kb + D);
                load_x(st[d].x, kb + D);
            }
        }
    }

    store_tiles<BN, TM, NF, MT>(acc, a, S, n_tile, m_tile, ks, n_tiles, m_tiles, wave * 16 * NF, 0);
}

template <int NF, int TM, int D>
static bool geom_mfma(const Variant& v, int M, int N, int K, dim3* grid, size_t* lds) {
    if (K <= 0) return false;
    constexpr int BN = 64 * NF;
    const int S = v.cfg.split;
    const int m_tiles = (M + TM - 1) / TM;
    if (TM > 16 && M <= TM / 2) return false;    // a smaller token tile fits
    const int n_tiles = (N + BN - 1) / BN;
    const int nkb = (K + kBK - 1) / kBK;
    if (S > 1 && nkb < 2 * S) return false;      // at least two k-blocks per split
    if (S > 1 && m_tiles * n_tiles > kMaxTileCounters) return false;
    *grid = dim3(tile_grid(n_tiles, m_tiles, S));
    *lds = 0;
    return true;
}

template <int NF, int TM, int D>
static size_t ws_mfma(const Variant& v, int M, int N, int K) {
    (void)K;
    const int S = v.cfg.split;
    if (S <= 1) return 0;
    constexpr int BN = 64 * NF;
    const size_t tiles = (size_t)((M + TM - 1) / TM) * ((N + BN - 1) / BN);
    return ws_counter_bytes((int)tiles) + (size_t)S * tiles * TM * BN * sizeof(float);
}

template <int NF, int TM, int D>
static void add(std::vector<Variant>& out, int S) {
    Variant v{};
    v.kind = LIN_KIND_SKINNY_BF16;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = 64 * NF;
    v.cfg.unroll = D;
    v.cfg.split = S;
    v.cfg.stage_x = 1;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = 16;
    v.func = (const void*)&gemm_mfma_kernel<NF, TM, D>;
    v.geometry = &geom_mfma<NF, TM, D>;
    v.workspace = &ws_mfma<NF, TM, D>;
    out.push_back(v);
}

template <int NF, int TM, int D>
static void add_splits(std::vector<Variant>& out) {
    for (int S : {1, 2, 4, 8, 16}) add<NF, TM, D>(out, S);
}

void register_gemm_mfma(std::vector<Variant>& out) {
    add_splits<1, 32, 4>(out);
    add_splits<1, 32, 8>(out);
    add_splits<1, 64, 2>(out);
    add_splits<1, 64, 4>(out);
    add_splits<2, 64, 4>(out);
    add_splits<1, 128, 2>(out);
    add_splits<1, 128, 4>(out);
    add_splits<2, 128, 2>(out);
    add_splits<2, 256, 2>(out);
}

}  // namespace lin

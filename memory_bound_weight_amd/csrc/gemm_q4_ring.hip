// Matrix-core product Y = X . W^T with int4-g64 weights, for batched decode
// (M <= 256 tokens), and the load-time rearrangement of the weights it reads.
//
// Why this shape.  4-bit weights make the batched product four times lighter
// on memory, so it reaches the matrix-core roof at a smaller batch; whether it
// then stays faster than bf16 depends on how cheaply the codes become
// matrix-core operands (llm-rs benchmark post, section 6: reordered weights at
// load time, one 16-byte load per lane handing it exactly its fragment, and a
// bit-trick conversion).  Here:
//  - Tiled weights.  lin_q4g64_tile rearranges Wq once so that one 1 KB
//    unit holds the codes of 16 rows x 128 k in operand order: lane l's 16
//    bytes are the four 8-code k-slices it feeds to the four 16x16x32 products
//    of that block (row l mod 16; k-step t covers 32 consecutive k inside one
//    scale group).  Inside a dword the codes of k0 + 2i and k0 + 2i + 1 sit at
//    bits 4i and 16 + 4i.  Scales are rearranged so that one 64-byte unit
//    holds the two groups of a 128-k block for 16 rows.
//  - Unpacking.  As in the GEMV (q4_unpack2): a dword of codes becomes bf16
//    pairs 24 + q (exact); with the nibble order of the tiles the pairs come
//    out in natural k order, so X is used as loaded.
//  - The offset and the scales.  The products of one scale group start from
//    C = -24 * sum(x) over the group, itself a matrix-core product of the X
//    operands with a constant operand of -24 (exact products, fp32 sums), so
//    D = sum(q x) for the group; then acc += s * D, one fma per output and
//    group.  Every product is exact in fp32 and the scale is applied in fp32:
//    nothing is rounded to bf16 on the way, unlike a dequantise-to-bf16 GEMM.
//  - Data path.  Codes, scales and X stream through an LDS ring of direct
//    global-to-LDS loads (gfx950 global_load_lds_dwordx4), D stages of one
//    128-k block, like the bf16 ring kernel; the codes are a quarter of the
//    bf16 bytes, so the ring mostly carries X.  X units are four token rows of
//    256 bytes, whole cache lines, with the 16-byte chunks of row r stored at
//    position c ^ r so that the operand reads of 16 rows spread over the banks.
//  - Tiles, split-K, tile order and the output store are those of the bf16
//    ring kernel (XCD-aware order, deterministic split-K).
#include "mfma_common.h"
#include "registry.h"

namespace lin {
namespace {

constexpr int kQB = 128;   // k per ring stage and per tiled unit

// bf16 pairs (-24, -24): the constant operand of the offset products.
constexpr uint32_t kNegOff = kQ4NegOffsetPair;

// Wave tile of a workgroup tile: NW wavefronts as WR x WC, as the bf16 ring
// except that eight wavefronts split a 128-token tile 4 x 2, not 2 x 4, and a
// 256 x 64 tile 8 x 1: every wavefront that reads a W fragment unpacks it, so
// fewer wavefronts across the tokens means less unpacking per product, at one
// offset product per NF fragments (M = 256, 32000x4096 with 256 x 128 tiles:
// 83 -> 77 us; 14336x4096 with 256 x 64 tiles: 43.5 -> 42.8 us).
template <int BN_, int TM_, int NW>
struct Q4Shape {
    static constexpr int BN = BN_, TM = TM_;
    static constexpr int WR = TM <= 16 ? NW : (NW == 4 ? (TM >= 256 ? 1 : 2) : (TM >= 256 ? 2 : (TM >= 128 || BN < 256 ? 4 : 8)));
    static constexpr int WC = NW / WR;
    static constexpr int WN = BN / WR, WM = TM / WC;
    static constexpr int NF = WN / 16, MT = WM / 16;
    static constexpr int FW = BN / 16;       // code units (1 KB) per stage
    static constexpr int FX = TM / 16 * 4;   // X units per stage (four token rows each)
    static constexpr int XU = FW + 1;        // first X unit; unit FW holds the scales
    static constexpr int F = (FW + 1 + FX + NW - 1) / NW * NW;   // units per stage, padded
    static constexpr int L = F / NW;         // units each wavefront loads per stage
    static_assert(NF >= 1 && MT >= 1 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(FW * 64 <= 1024, "the scales of a stage fit one unit");
};

// Two dwords of codes (two consecutive 8-k slices) to two B operands of bf16
// codes 24 + q; one v_bitop3 per pair, the shifts on both dwords at once.
__device__ __forceinline__ void unpack2(uint32_t w0, uint32_t w1, u32x4& b0, u32x4& b1) {
    uint32_t o[8];
    q4_unpack2((uint64_t)w0 | ((uint64_t)w1 << 32), o);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b0[i] = o[i];
        b1[i] = o[4 + i];
    }
}

__device__ __forceinline__ float half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Load unit u of a stage (code units 0 .. FW - 1, the scale unit FW, X units,
// then padding): a wavefront-uniform base at block 0, the bytes per block and
// the lane's byte offset from the base, and for X units the k of the lane's
// chunk within a block.  Row tiles past the last one re-read the last (their
// outputs are never stored); lanes of the scale unit past the workgroup's row
// tiles, and padding units, read bytes nobody uses.  Only X chunks past K must
// be zero: the last block of a K that is not a multiple of 128 takes the
// per-lane path with the zero word.
template <typename SH>
__device__ __forceinline__ void q4_unit(const KArgs& a, int u, int lane, int n_tile, int m_tile,
                                        const uint8_t*& base, int64_t& step, uint32_t& voff,
                                        int& kx) {
    constexpr int FW = SH::FW, FX = SH::FX, XU = SH::XU, BN = SH::BN, TM = SH::TM;
    const int M = a.M, N = a.N, K = a.K;
    const int N16 = (N + 15) >> 4;
    const int KBn = (K + kQB - 1) / kQB;
    const int T0 = n_tile * (BN / 16);
    base = (const uint8_t*)&g_zero16;
    step = 0;
    voff = 0;
    kx = 0;
    if (u < FW) {
        const int T = min(T0 + u, N16 - 1);
        base = (const uint8_t*)a.W + (int64_t)T * KBn * 1024;
        step = 1024;
        voff = 16 * lane;
    } else if (u == FW) {
        // lanes 4 f .. 4 f + 3 carry the 64-byte unit of row tile f
        base = (const uint8_t*)a.S + (int64_t)T0 * 64;
        step = (int64_t)N16 * 64;
        const int f = min(lane >> 2, FW - 1);
        voff = 64 * (min(T0 + f, N16 - 1) - T0) + 16 * (lane & 3);
    } else if (u < XU + FX) {
        const int x = u - XU;
        const int r = 4 * (x & 3) + (lane >> 4);   // token row within the 16-token tile
        const int c = (lane & 15) ^ r;             // chunk stored at position lane & 15
        int m = m_tile * TM + (x >> 2) * 16 + r;
        m = m < M ? m : M - 1;                     // rows past M: computed, never stored
        base = (const uint8_t*)a.X;
        step = kQB * 2;
        voff = (uint32_t)m * (uint32_t)K * 2u + 16u * c;
        kx = 8 * c;
    }
    base = uniform_ptr(base);
}

// The products of one ring stage for a wavefront: per scale group of 64 k,
// the offset products (X times the constant -24 operand), then for each W
// fragment the unpacked codes times X, scaled into the accumulators.
template <typename SH>
__device__ __forceinline__ void q4_stage_products(f32x4 (&acc)[SH::NF][SH::MT],
                                                  const u32x4 (*st)[64], int wr, int wc, int lane) {
    constexpr int NF = SH::NF, MT = SH::MT, FW = SH::FW, XU = SH::XU;
    const int l16 = lane & 15, lg = lane >> 4;
    const u32x4 neg = {kNegOff, kNegOff, kNegOff, kNegOff};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    u32x4 wq[NF];
    uint32_t sc[NF];
    const uint32_t* su = (const uint32_t*)&st[FW][0];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        wq[f] = st[wr * NF + f][lane];
        sc[f] = su[(wr * NF + f) * 16 + l16];
    }
    // X operand of token tile t, k-step q: row l16, chunk 4 q + lg.
    u32x4 ax[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const u32x4* xt = &st[XU + 4 * (wc * MT + t)][0];
#pragma unroll
        for (int q = 0; q < 4; ++q) ax[t][q] = xt[l16 * 16 + ((4 * q + lg) ^ l16)];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // the stage's two scale groups
        f32x4 cor[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            cor[t] = mfma16(ax[t][2 * h], neg, zero);
            cor[t] = mfma16(ax[t][2 * h + 1], neg, cor[t]);
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            u32x4 b0, b1;
            unpack2(wq[f][2 * h], wq[f][2 * h + 1], b0, b1);
            const float s = h ? half_hi(sc[f]) : half_lo(sc[f]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                f32x4 d = mfma16(ax[t][2 * h], b0, cor[t]);
                d = mfma16(ax[t][2 * h + 1], b1, d);
                acc[f][t] = d * s + acc[f][t];
            }
        }
    }
}

template <int BN, int TM, int D, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_q4_ring_kernel(KArgs a) {
    using SH = Q4Shape<BN, TM, NW>;
    constexpr int NF = SH::NF, MT = SH::MT, FX = SH::FX, XU = SH::XU, F = SH::F, L = SH::L;
    const int M = a.M, N = a.N, K = a.K;
    const int S = a.splits;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();

    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    int n_tile, m_tile, ks;
    if (!tile_of(blockIdx.x, n_tiles, m_tiles, S, n_tile, ks, m_tile))
        return;   // padding slot: the whole workgroup leaves together
    const int KBn = (K + kQB - 1) / kQB;   // 128-k blocks (units per row tile)
    const int bps = (KBn + S - 1) / S;
    const int kb0 = ks * bps;
    const int nkb = max(0, min(KBn, kb0 + bps) - kb0);

    __shared__ u32x4 ring[D][F][64];

    const uint8_t* base[L];
    int64_t step[L];
    uint32_t voff[L];
    int kx[L];   // X units: k of the lane's chunk within a block
#pragma unroll
    for (int i = 0; i < L; ++i)
        q4_unit<SH>(a, wave * L + i, lane, n_tile, m_tile, base[i], step[i], voff[i], kx[i]);
    const bool ktail = (K % kQB) != 0;
    auto issue = [&](int kb, int slot) {
        if (ktail && kb == KBn - 1) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int u = wave * L + i;
                const bool isx = u >= XU && u < XU + FX;
                const uint8_t* p = base[i] + kb * step[i] + voff[i];
                if (isx && kb * kQB + kx[i] >= K) p = (const uint8_t*)&g_zero16;
                dma16(p, &ring[slot][u][0]);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int u = wave * L + i;
            dma16s(base[i] + kb * step[i], voff[i], &ring[slot][u][0]);
        }
    };

    f32x4 acc[NF][MT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wr = wave / SH::WC, wc = wave - (wave / SH::WC) * SH::WC;
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (d < nkb) issue(kb0 + d, d);

    for (int i = 0; i < nkb; ++i) {
        wait_stages<L, D>(min(D - 2, nkb - 1 - i));   // stage i landed (own loads)
        ring_barrier();                                // everyone's loads of stage i landed
        if (i + D - 1 < nkb) issue(kb0 + i + D - 1, (i + D - 1) % D);
        q4_stage_products<SH>(acc, ring[i % D], wr, wc, lane);
    }

    store_tiles<BN, TM, NF, MT>(acc, a, S, n_tile, m_tile, ks, n_tiles, m_tiles, wr * SH::WN,
                                wc * SH::WM);
}


// The same product with NL loader wavefronts issuing every direct-to-LDS load
// (the protocol of the bf16 loader-wavefront ring): the NW product wavefronts
// only read operands, unpack and multiply, so none of them stalls on the load
// queue right after a barrier.
template <int BN, int TM, int D, int NW, int NL>
__global__ __launch_bounds__(64 * (NW + NL)) void gemm_q4_ring_ld_kernel(KArgs a) {
    using SH = Q4Shape<BN, TM, NW>;
    constexpr int NF = SH::NF, MT = SH::MT, FX = SH::FX, XU = SH::XU;
    constexpr int LL = (XU + FX + NL - 1) / NL;   // loads per loader and stage
    constexpr int FP = LL * NL;                    // units per stage, padded
    static_assert((D - 1) * LL < 64, "vmcnt range");
    const int M = a.M, N = a.N, K = a.K;
    const int S = a.splits;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();

    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    int n_tile, m_tile, ks;
    if (!tile_of(blockIdx.x, n_tiles, m_tiles, S, n_tile, ks, m_tile))
        return;   // padding slot: the whole workgroup leaves together
    const int KBn = (K + kQB - 1) / kQB;
    const int bps = (KBn + S - 1) / S;
    const int kb0 = ks * bps;
    const int nkb = max(0, min(KBn, kb0 + bps) - kb0);

    __shared__ u32x4 ring[D][FP][64];

    if (wave >= NW) {
        const int j = wave - NW;
        const uint8_t* base[LL];
        int64_t step[LL];
        uint32_t voff[LL];
        int kx[LL];
#pragma unroll
        for (int i = 0; i < LL; ++i)
            q4_unit<SH>(a, j * LL + i, lane, n_tile, m_tile, base[i], step[i], voff[i], kx[i]);
        const bool ktail = (K % kQB) != 0;
        auto issue = [&](int kb, int slot) {
            if (ktail && kb == KBn - 1) {
#pragma unroll
                for (int i = 0; i < LL; ++i) {
                    const int u = j * LL + i;
                    const bool isx = u >= XU && u < XU + FX;
                    const uint8_t* p = base[i] + kb * step[i] + voff[i];
                    if (isx && kb * kQB + kx[i] >= K) p = (const uint8_t*)&g_zero16;
                    dma16(p, &ring[slot][u][0]);
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < LL; ++i) dma16s(base[i] + kb * step[i], voff[i], &ring[slot][j * LL + i][0]);
        };
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (d < nkb) issue(kb0 + d, d);
        for (int i = 0; i < nkb; ++i) {
            wait_stages<LL, D>(min(D - 2, nkb - 1 - i));   // own loads of stage i landed
            ring_barrier();
            if (i + D - 1 < nkb) issue(kb0 + i + D - 1, (i + D - 1) % D);
        }
        if (S > 1) {   // the two barriers of the split-K store
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    f32x4 acc[NF][MT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wr = wave / SH::WC, wc = wave - (wave / SH::WC) * SH::WC;
    for (int i = 0; i < nkb; ++i) {
        wait_vm_lgkm<63, 0>();   // own operand reads of stage i - 1 complete
        ring_barrier();
        q4_stage_products<SH>(acc, ring[i % D], wr, wc, lane);
    }
    store_tiles<BN, TM, NF, MT>(acc, a, S, n_tile, m_tile, ks, n_tiles, m_tiles, wr * SH::WN,
                                wc * SH::WM);
}

template <int BN, int TM, int D, int NW>
bool geom_q4_ring(const Variant& v, int M, int N, int K, dim3* grid, size_t* lds) {
    if (K < 0) return false;
    if (TM > 16 && M <= TM / 2) return false;   // a smaller token tile fits
    const int S = v.cfg.split;
    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    const int nkb = (K + kQB - 1) / kQB;
    if (S > 1 && nkb < 2 * S) return false;      // at least two k-blocks per split
    if (S > 1 && m_tiles * n_tiles > kMaxTileCounters) return false;
    *grid = dim3(tile_grid(n_tiles, m_tiles, S));
    *lds = 0;
    return true;
}

template <int BN, int TM, int D, int NW>
size_t ws_q4_ring(const Variant& v, int M, int N, int K) {
    (void)K;
    const int S = v.cfg.split;
    if (S <= 1) return 0;
    const size_t tiles = (size_t)((M + TM - 1) / TM) * ((N + BN - 1) / BN);
    return ws_counter_bytes((int)tiles) + (size_t)S * tiles * TM * BN * sizeof(float);
}

template <int BN, int TM, int D, int NW = 4>
void add_q4(std::vector<Variant>& out, int S) {
    static_assert(D * Q4Shape<BN, TM, NW>::F * 1024 <= 160 * 1024, "LDS ring too large");
    Variant v{};
    v.kind = LIN_KIND_SKINNY_Q4G64;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = BN;
    v.cfg.unroll = D;
    v.cfg.split = S;
    v.cfg.stage_x = 4;   // everything through the LDS ring, X in whole lines
    v.cfg.waves = NW == 4 ? 0 : NW;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = 1;
    v.func = (const void*)&gemm_q4_ring_kernel<BN, TM, D, NW>;
    v.geometry = &geom_q4_ring<BN, TM, D, NW>;
    v.workspace = &ws_q4_ring<BN, TM, D, NW>;
    v.block = 64 * NW;
    out.push_back(v);
}

// Loader-wavefront form (stage_x 5): NW product wavefronts plus four loaders.
template <int BN, int TM, int D, int NW>
void add_q4_ld(std::vector<Variant>& out, int S) {
    constexpr int NL = 4;
    using SH = Q4Shape<BN, TM, NW>;
    constexpr int FP = (SH::XU + SH::FX + NL - 1) / NL * NL;
    static_assert(D * FP * 1024 <= 160 * 1024, "LDS ring too large");
    Variant v{};
    v.kind = LIN_KIND_SKINNY_Q4G64;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = BN;
    v.cfg.unroll = D;
    v.cfg.split = S;
    v.cfg.stage_x = 5;
    v.cfg.waves = NW == 4 ? 0 : NW;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = 1;
    v.func = (const void*)&gemm_q4_ring_ld_kernel<BN, TM, D, NW, NL>;
    v.geometry = &geom_q4_ring<BN, TM, D, NW>;
    v.workspace = &ws_q4_ring<BN, TM, D, NW>;
    v.block = 64 * (NW + NL);
    out.push_back(v);
}

// Tiled codes: one thread per lane of a unit (16 bytes).
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint8_t* __restrict__ Wq,
                                                         uint8_t* __restrict__ Wt, int N, int K) {
    const int KBn = (K + kQB - 1) / kQB;
    const int64_t units = (int64_t)((N + 15) >> 4) * KBn;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units * 64) return;
    const int l = (int)(i & 63);
    const int64_t unit = i >> 6;
    const int64_t T = unit / KBn;
    const int j = (int)(unit - T * KBn);
    const int64_t n = T * 16 + (l & 15);
    const int rowb = K / 2;   // bytes per plain row (a multiple of 32)
    u32x4 v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int off = 64 * j + 16 * t + 4 * (l >> 4);
        const uint32_t w = (n < N && off < rowb) ? *(const uint32_t*)(Wq + n * rowb + off) : 0u;
        // plain nibble e (k0 + e) at bits 4e -> even k at 4 (e / 2), odd at 16 + 4 (e / 2)
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) o |= ((w >> (4 * e)) & 0xFu) << ((e & 1) * 16 + 4 * (e >> 1));
        v[t] = o;
    }
    *(u32x4*)(Wt + i * 16) = v;
}

// Tiled scales: one thread per (block, row tile, row) = one dword (two fp16).
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint16_t* __restrict__ S,
                                                          uint32_t* __restrict__ St, int N, int K) {
    const int KBn = (K + kQB - 1) / kQB;
    const int N16 = (N + 15) >> 4;
    const int G = K / 64;
    const int64_t total = (int64_t)KBn * N16 * 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int r = (int)(i & 15);
    const int64_t unit = i >> 4;   // j * N16 + T
    const int j = (int)(unit / N16);
    const int64_t T = unit - (int64_t)j * N16;
    const int64_t n = T * 16 + r;
    uint32_t lo = 0, hi = 0;
    if (n < N) {
        if (2 * j < G) lo = S[n * G + 2 * j];
        if (2 * j + 1 < G) hi = S[n * G + 2 * j + 1];
    }
    St[i] = lo | (hi << 16);
}

}  // namespace

void q4g64_tiled_bytes(int64_t N, int64_t K, int64_t* wt, int64_t* st) {
    const int64_t n16 = (N + 15) / 16, kb = (K + kQB - 1) / kQB;
    *wt = n16 * kb * 1024;
    *st = n16 * kb * 64;
}

hipError_t launch_tile_q4g64(const void* Wq, const void* S, void* Wt, void* St, int N, int K,
                             hipStream_t stream) {
    const int64_t n16 = (N + 15) / 16, kb = (K + kQB - 1) / kQB;
    const int64_t code_threads = n16 * kb * 64;
    const int64_t scale_threads = n16 * kb * 16;
    if (code_threads > 0) {
        hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((code_threads + 255) / 256)), dim3(256),
                           0, stream, (const uint8_t*)Wq, (uint8_t*)Wt, N, K);
        hipLaunchKernelGGL(tile_scales_kernel, dim3((unsigned)((scale_threads + 255) / 256)),
                           dim3(256), 0, stream, (const uint16_t*)S, (uint32_t*)St, N, K);
    }
    return hipGetLastError();
}

void register_gemm_q4_ring(std::vector<Variant>& out) {
    for (int S : {1, 2, 4, 8}) {
        add_q4<64, 16, 6>(out, S);
        add_q4<128, 16, 6>(out, S);
        add_q4<256, 16, 4>(out, S);
        add_q4<64, 32, 6>(out, S);
        add_q4<128, 32, 4>(out, S);
        add_q4<64, 64, 4>(out, S);
        add_q4<128, 64, 4>(out, S);
        add_q4<128, 64, 3>(out, S);
        add_q4<64, 128, 3>(out, S);
        add_q4<128, 128, 3>(out, S);
        add_q4<128, 128, 2>(out, S);
        add_q4<64, 256, 2>(out, S);
        add_q4<256, 128, 3>(out, S);
        add_q4<256, 128, 2>(out, S);
        add_q4<256, 64, 4>(out, S);
        // eight wavefronts, two per SIMD: one multiplies while the other unpacks
        add_q4<128, 16, 6, 8>(out, S);
        add_q4<128, 64, 4, 8>(out, S);
        add_q4<256, 64, 3, 8>(out, S);
        add_q4<128, 128, 3, 8>(out, S);
        add_q4<128, 128, 2, 8>(out, S);
        add_q4<256, 128, 2, 8>(out, S);
        add_q4<64, 256, 2, 8>(out, S);
        add_q4_ld<64, 16, 6, 4>(out, S);
        add_q4_ld<128, 16, 6, 4>(out, S);
        add_q4_ld<128, 16, 6, 8>(out, S);
        add_q4_ld<64, 32, 6, 4>(out, S);
        add_q4_ld<128, 32, 4, 4>(out, S);
        add_q4_ld<64, 64, 4, 4>(out, S);
        add_q4_ld<128, 64, 4, 4>(out, S);
        add_q4_ld<128, 64, 4, 8>(out, S);
        add_q4_ld<256, 64, 3, 8>(out, S);
        add_q4_ld<64, 128, 3, 4>(out, S);
        add_q4_ld<128, 128, 3, 8>(out, S);
        add_q4_ld<128, 128, 2, 8>(out, S);
    }
}

}  // namespace lin

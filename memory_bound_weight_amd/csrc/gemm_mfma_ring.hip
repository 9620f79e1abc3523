// Matrix-core product Y = X . W^T with both operands streamed through an LDS
// ring filled by direct-to-LDS loads (gfx950 global_load_lds_dwordx4).
//
// Why.  Batched decode keeps the product memory-bound up to a few hundred
// tokens (llm-rs benchmark post, section 3), so what matters is how many
// weight bytes each compute unit keeps in flight: under full load HBM
// latency is several microseconds, and a register ring of a few k-blocks per
// workgroup leaves the chip latency-bound.  A direct-to-LDS load moves 16
// bytes per lane from memory into LDS without passing through registers, so
// the ring depth is bounded by the 160 KB of LDS instead of the register
// file, and the loads of D k-blocks are in flight at once.  Pipelining and
// bank-conflict-free staging follow section 5 of the same post; the data
// path is CDNA4's own.
//
// Ring.  A stage holds one 64-k block of BN W rows and TM X rows in 1 KB
// load units, one wavefront instruction (64 lanes x 16 B, placed in lane
// order) each.  Two unit layouts:
//  - fragment order: a unit is 16 rows x 64 B (32 k), in the order
//    v_mfma_f32_16x16x32_bf16 reads its operands (lane l: row l mod 16, k
//    8 (l / 16) .. + 7), read back with one lane-linear ds_read_b128;
//  - line order: a unit is 8 rows x 128 B, whole cache lines, with the 16-byte
//    chunks of a row XOR-swizzled so that the operand reads of a 16-row group
//    (two units) are still one ds_read_b128 spread over the banks.  Half as
//    many cache lines per load instruction: X, which every workgroup re-reads
//    from L2, streams faster (measured 40 %), at a small cost in LDS reads.
// The wavefronts share the loads of a stage.  Iteration i waits (vmcnt)
// until its own loads of stage i have landed, meets the others at one
// s_barrier (their loads have landed too, and everyone has finished reading
// stage i - 1), refills the slot of stage i - 1 with stage i + D - 1, then
// multiplies stage i.  k past K reads from a zero word, rows past N or M
// re-read the last row (never stored); the loads take a wavefront-uniform
// base in SGPRs and a per-lane offset, so moving to the next stage is a
// scalar add.
//
// Wave tile.  The workgroup tile BN x TM is split 2 x 2 (or 1 x 4 when TM is
// 256) among four wavefronts, or 2 x 4 / 4 x 2 among eight (two per SIMD,
// so one can multiply while the other waits), or 1 x NW when the tile's
// 16-row fragments do not split evenly (112-row tiles); each keeps its NF x MT
// 16x16 fp32 accumulators in registers and writes them directly, or as a
// split-K partial that the last workgroup of the tile adds in split order
// (deterministic).
//
// A second kernel below adds loader wavefronts that issue every load of the
// ring, so that the product wavefronts never stall on the load queue.
#include "mfma_common.h"
#include "registry.h"

namespace lin {
namespace {

// Position of k-chunk c (8 k, 16 bytes) in row r of a ring group is
// c ^ ring_swz(r).  The 16 rows of a group are 128 bytes apart, so unswizzled
// the 16 lanes reading one chunk of 16 rows would hit the same banks (measured
// 12 conflict cycles per ds_read_b128).  XOR with the row modulo 8 gives any 8
// consecutive rows 8 different 16-byte positions; measured on gfx950 that is
// conflict-free for both 32-k halves.  Also folding in bit 3 of the row (so
// that all 16 rows differ within 256 bytes) measured 4 conflict cycles per
// read instead: the banks are not simply the low address bits.
__device__ __forceinline__ int ring_swz(int r) { return r & 7; }

// The ring's direct-to-LDS loads use dma16 (ordinary cache policy: a
// non-temporal hint on the weights measured slower); k >= K lanes load
// g_zero16 instead of reading past a row.

// Wave tile of a workgroup tile: NW wavefronts as WR x WC; KB k per stage
// (eight wavefronts and 128-k stages measured no faster than 4 and 64).  A
// 16-token tile stacks the wavefronts along W (4 x 1).  The fragment loads of
// a stage are spread evenly over the wavefronts; when their number does not
// divide, the stage is padded with fragments that load the zero word.
template <int BN, int TM, int NW, int KB>
struct Shape {
    static constexpr int WR0 = TM <= 16 ? NW : (NW == 4 ? (TM >= 256 ? 1 : 2) : (TM >= 128 ? 2 : 4));
    // a tile whose 16-row fragments do not split WR0 ways stacks the wavefronts along the tokens
    static constexpr int WR = (BN / 16) % WR0 == 0 ? WR0 : 1;
    static constexpr int WC = NW / WR;
    static constexpr int WN = BN / WR, WM = TM / WC;
    static constexpr int NF = WN / 16, MT = WM / 16;
    static constexpr int H = KB / 32;                  // 32-k halves per stage
    static constexpr int FW = BN / 16 * H, FX = TM / 16 * H;
    static constexpr int F = (FW + FX + NW - 1) / NW * NW;   // fragments per stage, padded
    static constexpr int L = F / NW;                   // fragment loads per wavefront and stage
    static_assert(NF >= 1 && MT >= 1 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(KB == 64, "a ring group is 16 rows x 128 bytes");
};

// Load unit u of a stage (W units 0 .. FW - 1, then X units, then padding):
// a wavefront-uniform base (the first row of the unit's 16-row group,
// clamped), the lane's byte offset from it and its k within a block, and the
// bytes per block (0 for padding, which re-reads the zero word).  Fragment
// order: unit u is half u % 2 of 16-row group u / 2, lane l takes row l % 16
// and k 32 (u % 2) + 8 (l / 16).  Line order: unit u is rows 8 (u % 2) .. + 7
// of group u / 2, lane l takes row 8 (u % 2) + l / 8 and stores, at position
// l % 8 of that row, k-chunk (l % 8) ^ swz(row).
template <int BN, int TM, int FW, int FX, int KB, bool LINE>
__device__ __forceinline__ void ring_unit(const KArgs& a, int u, int lane, int n_tile, int m_tile,
                                          const uint8_t*& base, uint32_t& voff, int& koff,
                                          int& step) {
    const int N = a.N, M = a.M, K = a.K;
    const int r = LINE ? (u & 1) * 8 + (lane >> 3) : (lane & 15);   // row within the group
    koff = LINE ? ((lane & 7) ^ ring_swz(r)) * 8 : (u & 1) * 32 + (lane >> 4) * 8;
    base = (const uint8_t*)&g_zero16;
    voff = 0;
    step = 0;
    if (u < FW + FX) {
        const bool isw = u < FW;
        const int lim = isw ? N : M;
        const int g0 = isw ? n_tile * BN + (u >> 1) * 16 : m_tile * TM + ((u - FW) >> 1) * 16;
        const int r0 = min(g0, lim - 1);
        const int row = min(g0 + r, lim - 1);   // rows past the end: computed, never stored
        base = (const uint8_t*)(isw ? a.W : a.X) + (int64_t)r0 * K * 2;
        voff = (uint32_t)(row - r0) * (uint32_t)K * 2u + 2u * koff;
        step = KB * 2;
    }
    base = uniform_ptr(base);
}

// The products of one ring stage for a wavefront: its NF W fragments and MT
// X fragments of both 32-k halves, read from the stage's units, then H x NF x
// MT products.  Operand of lane l for half h of a 16-row group: fragment
// order, entry l of unit 2 g + h; line order, row l % 16 of the group at
// position (4 h + l / 16) ^ swz(row) (the two units of the group are
// contiguous).  All operand reads of the stage are issued up front; the
// scheduler is then asked to interleave the reads of the second half with the
// products of the first, so that their LDS latency overlaps the matrix cores
// instead of stalling in front of them.
template <typename SH, bool LINE>
__device__ __forceinline__ void stage_products(f32x4 (&acc)[SH::NF][SH::MT], const u32x4 (*st)[64],
                                               int wr, int wc, int lane) {
    constexpr int NF = SH::NF, MT = SH::MT, H = SH::H, FW = SH::FW;
    const int l16 = lane & 15, lg = lane >> 4;
    const int rsw = ring_swz(l16);
    auto operand = [&](int unit0, int h) -> u32x4 {
        if constexpr (LINE)
            return (&st[unit0][0])[l16 * 8 + ((4 * h + lg) ^ rsw)];
        else
            return st[unit0 + h][lane];
    };
    u32x4 bw[H][NF], ax[H][MT];
#pragma unroll
    for (int h = 0; h < H; ++h) {
#pragma unroll
        for (int f = 0; f < NF; ++f) bw[h][f] = operand(2 * (wr * NF + f), h);
#pragma unroll
        for (int t = 0; t < MT; ++t) ax[h][t] = operand(FW + 2 * (wc * MT + t), h);
    }
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[f][t] = mfma16(ax[h][t], bw[h][f], acc[f][t]);
    // first half's reads, then one read of the second half per product
    __builtin_amdgcn_sched_group_barrier(0x100, NF + MT, 0);
#pragma unroll
    for (int q = 0; q < (H - 1) * (NF + MT); ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, H * NF * MT - (H - 1) * (NF + MT), 0);
}

template <int BN, int TM, int D, int NW, int KB, bool LINE>
__global__ __launch_bounds__(64 * NW) void gemm_mfma_ring_kernel(KArgs a) {
    using SH = Shape<BN, TM, NW, KB>;
    constexpr int NF = SH::NF, MT = SH::MT, FW = SH::FW, F = SH::F, L = SH::L;
    const int M = a.M, N = a.N, K = a.K;
    const int S = a.splits;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();

    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    int n_tile, m_tile, ks;
    if (!tile_of(blockIdx.x, n_tiles, m_tiles, S, n_tile, ks, m_tile))
        return;   // padding slot: the whole workgroup leaves together
    const int nkb_all = (K + KB - 1) / KB;
    const int bps = (nkb_all + S - 1) / S;
    const int kb0 = ks * bps;
    const int nkb = max(0, min(nkb_all, kb0 + bps) - kb0);

    __shared__ u32x4 ring[D][F][64];

    // Load units this wavefront issues per stage: u = wave * L + i.
    // Steady-state loads use the scalar-base form with no per-lane address
    // arithmetic; only the last block of a K that is not a multiple of KB
    // checks each chunk against K (k >= K loads the zero word).  Padding units
    // read bytes nobody uses.
    const uint8_t* base[L];
    uint32_t voff[L];
    int koff[L];
    int step[L];
#pragma unroll
    for (int i = 0; i < L; ++i)
        ring_unit<BN, TM, FW, SH::FX, KB, LINE>(a, wave * L + i, lane, n_tile, m_tile, base[i],
                                                voff[i], koff[i], step[i]);
    const bool ktail = (K % KB) != 0;
    auto issue = [&](int kb, int slot) {
        if (ktail && kb == nkb_all - 1) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int u = wave * L + i;
                const uint8_t* p = base[i] + (int64_t)kb * step[i] + voff[i];
                if (kb * KB + koff[i] >= K) p = (const uint8_t*)&g_zero16;   // K % 8 == 0
                dma16(p, &ring[slot][u][0]);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int u = wave * L + i;
            dma16s(base[i] + (int64_t)kb * step[i], voff[i], &ring[slot][u][0]);
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
        stage_products<SH, LINE>(acc, ring[i % D], wr, wc, lane);
    }

    // Output: lane holds W row n_tile BN + wr WN + 16 f + l16, tokens
    // m_tile TM + wc WM + 16 t + 4 lg + r.
    store_tiles<BN, TM, NF, MT>(acc, a, S, n_tile, m_tile, ks, n_tiles, m_tiles, wr * SH::WN,
                                wc * SH::WM);
}


// Ring with loader wavefronts.  The direct-to-LDS loads of a stage are issued
// by NL wavefronts of their own; the NW product wavefronts only read
// operands and multiply.  A load instruction does not leave the issuing
// wavefront until the compute unit's load path accepts it (about 1 KB per 16
// cycles), so in the ring above every wavefront stalls for its share of that
// queue right after the barrier, in lockstep with the others, and the matrix
// cores idle meanwhile; here those stalls fall on wavefronts that have no
// products to hold up.  Per iteration i (every wavefront meets every
// barrier): a loader waits until its own loads of stage i have landed, meets
// the barrier, then refills the slot of stage i - 1 with stage i + D - 1; a
// product wavefront waits for its own operand reads of stage i - 1, meets the
// barrier (stage i has landed, nobody still reads stage i - 1), then
// multiplies stage i.  For split-K the loaders also meet the two barriers of
// the store.
template <int BN, int TM, int D, int NW, int NL>
__global__ __launch_bounds__(64 * (NW + NL)) void gemm_mfma_ring_ld_kernel(KArgs a) {
    constexpr int KB = 64;
    using SH = Shape<BN, TM, NW, KB>;
    constexpr int NF = SH::NF, MT = SH::MT, FW = SH::FW, FX = SH::FX;
    constexpr int LL = (FW + FX + NL - 1) / NL;   // loads per loader and stage
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
    const int nkb_all = (K + KB - 1) / KB;
    const int bps = (nkb_all + S - 1) / S;
    const int kb0 = ks * bps;
    const int nkb = max(0, min(nkb_all, kb0 + bps) - kb0);

    __shared__ u32x4 ring[D][FP][64];

    if (wave >= NW) {
        const int j = wave - NW;
        const uint8_t* base[LL];
        uint32_t voff[LL];
        int koff[LL];
        int step[LL];
#pragma unroll
        for (int i = 0; i < LL; ++i)
            ring_unit<BN, TM, FW, FX, KB, true>(a, j * LL + i, lane, n_tile, m_tile, base[i], voff[i],
                                                koff[i], step[i]);
        const bool ktail = (K % KB) != 0;
        auto issue = [&](int kb, int slot) {
            if (ktail && kb == nkb_all - 1) {
#pragma unroll
                for (int i = 0; i < LL; ++i) {
                    const uint8_t* p = base[i] + (int64_t)kb * step[i] + voff[i];
                    if (kb * KB + koff[i] >= K) p = (const uint8_t*)&g_zero16;   // K % 8 == 0
                    dma16(p, &ring[slot][j * LL + i][0]);
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < LL; ++i)
                dma16s(base[i] + (int64_t)kb * step[i], voff[i], &ring[slot][j * LL + i][0]);
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
        stage_products<SH, true>(acc, ring[i % D], wr, wc, lane);
    }
    store_tiles<BN, TM, NF, MT>(acc, a, S, n_tile, m_tile, ks, n_tiles, m_tiles, wr * SH::WN,
                                wc * SH::WM);
}

template <int BN, int TM, int D, int NW, int KB>
bool geom_ring(const Variant& v, int M, int N, int K, dim3* grid, size_t* lds) {
    if (K <= 0) return false;
    if (TM > 32 && M <= TM / 2) return false;   // a smaller token tile fits
    const int S = v.cfg.split;
    const int m_tiles = (M + TM - 1) / TM;
    const int n_tiles = (N + BN - 1) / BN;
    const int nkb = (K + KB - 1) / KB;
    if (S > 1 && nkb < 2 * S) return false;      // at least two k-blocks per split
    if (S > 1 && m_tiles * n_tiles > kMaxTileCounters) return false;
    *grid = dim3(tile_grid(n_tiles, m_tiles, S));
    *lds = 0;
    return true;
}

template <int BN, int TM, int D, int NW, int KB>
size_t ws_ring(const Variant& v, int M, int N, int K) {
    (void)K;
    const int S = v.cfg.split;
    if (S <= 1) return 0;
    const size_t tiles = (size_t)((M + TM - 1) / TM) * ((N + BN - 1) / BN);
    return ws_counter_bytes((int)tiles) + (size_t)S * tiles * TM * BN * sizeof(float);
}

template <int BN, int TM, int D, bool LINE, int NW = 4, int KB = 64>
void add_ring1(std::vector<Variant>& out, int S) {
    // the ring plus the split-K flag must fit the 160 KB of LDS
    static_assert(D * Shape<BN, TM, NW, KB>::F * 1024 < 160 * 1024, "LDS ring too large");
    Variant v{};
    v.kind = LIN_KIND_SKINNY_BF16;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = BN;
    v.cfg.unroll = D;
    v.cfg.split = S;
    // W and X blocks through an LDS ring of direct loads: 3 fragment order,
    // 4 line order
    v.cfg.stage_x = LINE ? 4 : 3;
    v.cfg.waves = NW == 4 ? 0 : NW;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = TM <= 16 ? 1 : 16;
    v.func = (const void*)&gemm_mfma_ring_kernel<BN, TM, D, NW, KB, LINE>;
    v.geometry = &geom_ring<BN, TM, D, NW, KB>;
    v.workspace = &ws_ring<BN, TM, D, NW, KB>;
    v.block = 64 * NW;
    out.push_back(v);
}

// Loader-wavefront ring (stage_x 5): NW product wavefronts (`waves`, 0 for
// four) plus four loader wavefronts, line order.
template <int BN, int TM, int D, int NW>
void add_ring_ld(std::vector<Variant>& out, int S) {
    constexpr int NL = 4;
    using SH = Shape<BN, TM, NW, 64>;
    constexpr int FP = (SH::FW + SH::FX + NL - 1) / NL * NL;
    static_assert(D * FP * 1024 < 160 * 1024, "LDS ring too large");
    Variant v{};
    v.kind = LIN_KIND_SKINNY_BF16;
    v.cfg.algo = LIN_ALGO_MFMA;
    v.cfg.rows = BN;
    v.cfg.unroll = D;
    v.cfg.split = S;
    v.cfg.stage_x = 5;
    v.cfg.waves = NW == 4 ? 0 : NW;
    v.cfg.tile_m = TM;
    v.mt = 0;
    v.min_m = TM <= 16 ? 1 : 16;
    v.func = (const void*)&gemm_mfma_ring_ld_kernel<BN, TM, D, NW, NL>;
    v.geometry = &geom_ring<BN, TM, D, NW, 64>;
    v.workspace = &ws_ring<BN, TM, D, NW, 64>;
    v.block = 64 * (NW + NL);
    out.push_back(v);
}

template <int BN, int TM, int D>
void add_ring(std::vector<Variant>& out, int S) {
    add_ring1<BN, TM, D, false>(out, S);
    add_ring1<BN, TM, D, true>(out, S);
}

}  // namespace

void register_gemm_mfma_ring(std::vector<Variant>& out) {
    for (int S : {1, 2, 4, 8}) {
        add_ring<64, 16, 8>(out, S);
        add_ring<128, 16, 6>(out, S);
        add_ring<32, 32, 8>(out, S);
        add_ring<32, 64, 6>(out, S);
        add_ring<64, 32, 8>(out, S);
        add_ring<64, 64, 4>(out, S);
        add_ring<64, 128, 4>(out, S);
        add_ring<128, 64, 4>(out, S);
        add_ring<64, 256, 3>(out, S);
        add_ring<128, 128, 4>(out, S);
        add_ring<128, 128, 2>(out, S);
        add_ring<64, 128, 3>(out, S);
        add_ring<128, 64, 3>(out, S);
        add_ring1<128, 128, 4, true, 8>(out, S);
        add_ring1<128, 128, 2, true, 8>(out, S);
        add_ring1<64, 64, 4, true, 8>(out, S);
        add_ring1<128, 64, 4, true, 8>(out, S);
        add_ring1<128, 64, 3, true, 8>(out, S);
        add_ring1<256, 64, 3, true, 8>(out, S);
        add_ring1<128, 128, 3, true, 8>(out, S);
        add_ring1<256, 128, 3, true, 8>(out, S);
        add_ring1<256, 128, 3, true, 4>(out, S);
        add_ring1<64, 128, 5, true, 8>(out, S);
        add_ring_ld<64, 16, 8, 4>(out, S);
        add_ring_ld<128, 16, 6, 4>(out, S);
        add_ring_ld<32, 32, 8, 4>(out, S);
        add_ring_ld<64, 32, 8, 4>(out, S);
        add_ring_ld<64, 64, 4, 4>(out, S);
        add_ring_ld<64, 64, 6, 4>(out, S);
        add_ring_ld<64, 64, 4, 8>(out, S);
        add_ring_ld<128, 64, 4, 4>(out, S);
        add_ring_ld<128, 64, 4, 8>(out, S);
        add_ring_ld<128, 128, 3, 4>(out, S);
        add_ring_ld<128, 128, 4, 4>(out, S);
        add_ring_ld<128, 128, 3, 8>(out, S);
        add_ring_ld<128, 128, 4, 8>(out, S);
        add_ring_ld<256, 64, 3, 8>(out, S);
        add_ring_ld<256, 128, 3, 4>(out, S);
        add_ring_ld<256, 128, 3, 8>(out, S);
        add_ring_ld<128, 256, 3, 8>(out, S);
        add_ring_ld<64, 256, 3, 4>(out, S);
        add_ring_ld<64, 256, 3, 8>(out, S);
        add_ring1<112, 128, 4, true, 4>(out, S);
        add_ring1<112, 128, 4, true, 8>(out, S);
        add_ring_ld<112, 128, 4, 4>(out, S);
        add_ring_ld<112, 128, 4, 8>(out, S);
    }
}

}  // namespace lin

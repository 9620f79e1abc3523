// int4-g64 batch-1 product with x resident in registers: the wavefront streams
// many rows through a prefetch pipeline (a second kernel family for
// lin_gemv_q4g64, selected by tuning; configuration stage_x = 2, `rows` = the
// outputs per wavefront group, `unroll` = rows in flight, `split` = KS).
//
// Why.  The wavefront-per-R-rows kernel (gemv_q4g64_impl.h) re-reads x for
// every R rows: each lane's 16 bytes of codes need 64 bytes of x, four
// 16-byte loads that touch four times as many cache lines as the codes, and
// every wavefront makes one round of loads and then computes, so a launch
// runs as a few waves of long-latency rounds.  Here the reduction dimension
// is cut once per wavefront, not per row: the row's nch 32-code chunks are
// split into KS equal contiguous slices of C = ceil(nch / KS) chunks, one per
// wavefront of a row group, and lane l of the part-th wavefront owns the
// chunks part * C + l + 64 j (j < J, l + 64 j < C) of every row, so the
// wavefronts of a group stream equal bytes.  It loads and re-pairs
// the x of those chunks once (pair_x: 16 dwords and -24 sum x per chunk) and
// keeps them in registers; then it walks its rows, keeping P rows of codes and
// scales in flight (16-byte code loads, 2-byte scale loads), so the main loop
// issues only weight loads (tinyinfer post, v0.2: more independent 16-byte
// loads in flight per warp; here they come from later rows rather than from
// more rows at once).
//
// Products are the GEMV's: exact bf16 codes 24 + q (q4_unpack2), dot2 with the
// paired x from -24 sum x, times the group scale in fp32.  The per-lane row
// sums are reduced across the wavefront P rows at a time; KS > 1 adds the
// parts through LDS in a fixed order.
//
// Rows: the grid has ng = GROUPS * ceil(N / (GROUPS * RW)) groups (rounded
// up to whole compute units) and group g takes the contiguous outputs
// N g / ng .. N (g + 1) / ng - 1, at most RW, so every group streams the same
// number of rows (+-1) for any N, and each streams one contiguous block of
// the matrix (interleaving the groups' rows so that all groups read one
// sliding window was measured slower).  Group numbers follow the XCD the
// workgroup runs on, so each XCD streams one contiguous eighth of the rows
// (1-2 % faster on the 7B shapes: fewer scale lines fetched twice).  The loop
// over RW rows is unrolled (every wait an exact immediate count, no branches
// that would make the compiler drain the pipeline); a group with fewer rows
// reads its missing rows past the end of its buffer resource, which returns
// zeros without touching memory, and drops them.
//
// Epilogues as the other GEMV kernels: the residual add, and the gated
// product over gate|up, where an output needs its gate row and its up row
// (both streamed, totals meeting in LDS).
#include "gemv_q4g64_impl.h"
#include "registry.h"

namespace lin {

// Buffer resource over `bytes` bytes from `base` (raw, no stride; reads past
// the end return 0 without a memory access).  Row loads take the row offset
// in an SGPR and the lane offset in a VGPR: the row bases never become
// per-lane addresses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t q4x_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
constexpr int kNontemporal = 2;   // buffer-load cache policy: streaming (nt)

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }

// Rows in flight for epilogue EPI when the plain product keeps P in flight:
// the gated product streams two weight rows per output, so it keeps fewer in
// flight where the wait counter (at most 63 loads) or the registers (about 60
// for the stages next to the resident x) would not hold P.
template <int J, int P, int EPI>
constexpr int q4x_depth() {
    constexpr int NR = EPI == kEpiSwiglu ? 2 : 1;
    int d = P;
    while (d > 1 && (d * 2 * NR * J > 63 || (NR > 1 && d * NR * J * 5 > 60))) d /= 2;
    return d;
}

template <int J, int KS, int P0, int RW, int EPI>
__global__ __launch_bounds__(kBlock) void gemv_q4_xres(KArgs a) {
    static_assert(KS == 1 || KS == 2 || KS == 4, "K slices per row group");
    constexpr int P = q4x_depth<J, P0, EPI>();
    constexpr int NR = EPI == kEpiSwiglu ? 2 : 1;    // weight rows per output
    constexpr int V = pow2_at_least(RW * NR);        // row totals reduced at once
    constexpr int LPI = 2 * NR * J;                  // loads per output (codes, scales)
    static_assert(P >= 1 && P * LPI <= 63 && V <= 64, "pipeline shape");
    constexpr int GROUPS = 4 / KS;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = wave / KS;
    const int part = wave - grp * KS;
    const int N = a.N, K = a.K;
    const int nch = K >> 5;
    const int G = K >> 6;
    const int rowb = K / 2;   // code bytes per row
    const uint8_t* __restrict__ Wq = (const uint8_t*)a.W;
    const uint16_t* __restrict__ S = (const uint16_t*)a.S;
    const uint8_t* __restrict__ X = (const uint8_t*)a.X;

    // this group's outputs: a balanced contiguous share (at most RW) of the N
    // floor(N g / ng) for g = gi, gi + 1.  With N = q ng + r that is
    // q g + floor(r g / ng), whose products fit 32 bits while ng < 2^16 (every
    // shape here); the 64-bit division it replaces is a few hundred scalar
    // instructions in front of the first load of every wavefront.
    const uint32_t ng = gridDim.x * GROUPS;
    // Workgroups go round-robin over the eight XCDs: hand XCD x the x-th
    // eighth of the row groups, so that the scale-row line two neighbouring
    // groups share is fetched into one XCD's L2, not two (a bijection on the
    // workgroup index; the grid is a whole number of compute units).
    const uint32_t nb = gridDim.x;
    const uint32_t bx = (nb & 7u) == 0 ? (blockIdx.x & 7u) * (nb >> 3) + (blockIdx.x >> 3)
                                       : blockIdx.x;
    const uint32_t gi = bx * GROUPS + grp;
    int o0, o1;
    if (ng < 65536u) {
        const uint32_t q = (uint32_t)N / ng, r = (uint32_t)N - q * ng;
        o0 = (int)(q * gi + r * gi / ng);
        o1 = (int)(q * (gi + 1) + r * (gi + 1) / ng);
    } else {
        o0 = (int)((int64_t)N * gi / ng);
        o1 = (int)((int64_t)N * (gi + 1) / ng);
    }
    const int n_out = o1 - o0;

    // the lane's chunks (clamped to the last chunk; their products are dropped)
    const int C = (nch + KS - 1) / KS;   // chunks per slice
    uint32_t coff[J], soff[J];
    bool ok[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int cl = lane + kWave * j;   // chunk within the slice
        const int c = part * C + cl;
        ok[j] = cl < C && c < nch;
        const int cc = c < nch ? c : nch - 1;
        coff[j] = (uint32_t)cc * 16u;
        soff[j] = (uint32_t)(cc >> 1) * 2u;
    }

    // x of the lane's chunks: issued first, re-paired once the first rows'
    // weight loads are in flight
    u32x4 xraw[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) xraw[j][t] = load_x16(X, coff[j] * 4u + 16u * t);

    // one resource per weight-row set of this group (the outputs' rows and,
    // for the gated product, their up rows N further), codes and scales
    const int wstride = rowb, sstride = G * 2;   // bytes between this group's rows
    __amdgpu_buffer_rsrc_t rw[NR], rs[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t first = (int64_t)o0 + (r ? (int64_t)N : 0);
        rw[r] = q4x_rsrc(Wq + first * rowb, n_out * wstride);
        rs[r] = q4x_rsrc(S + first * G, n_out * sstride);
    }
    u32x4 w[P][NR][J];
    uint16_t sc[P][NR][J];
    // The scheduling barriers keep every row's loads where they are issued
    // (left free, the scheduler may sink them next to their products).
    auto issue = [&](int s, int i) {   // output o0 + i (past n_out: zeros, no access)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                w[s][r][j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw[r], (int)coff[j], i * wstride,
                                                                 kNontemporal));
                sc[s][r][j] = __builtin_amdgcn_raw_buffer_load_b16(rs[r], (int)soff[j],
                                                                   i * sstride, kNontemporal);
            }
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int PRE = P < RW ? P : RW;
#pragma unroll
    for (int i = 0; i < PRE; ++i) issue(i, i);
    wait_cnt<PRE * LPI, 15>();   // the x loads have landed (loads complete in order)
    XChunk xr[J];
#pragma unroll
    for (int j = 0; j < J; ++j) pair_x(xraw[j], xr[j]);

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int s = i % P;
        // outputs i+1 .. min(i+P-1, RW-1) (those issued) may still be in flight
        const int ahead = (RW - 1 - i) < (P - 1) ? (RW - 1 - i) : (P - 1);
        switch (ahead) {   // a constant after unrolling: no branch remains
            case 0: wait_cnt<0, 15>(); break;
            case 1: wait_cnt<1 * LPI, 15>(); break;
            case 2: wait_cnt<(2 * LPI < 63 ? 2 * LPI : 63), 15>(); break;
            case 3: wait_cnt<(3 * LPI < 63 ? 3 * LPI : 63), 15>(); break;
            case 4: wait_cnt<(4 * LPI < 63 ? 4 * LPI : 63), 15>(); break;
            case 5: wait_cnt<(5 * LPI < 63 ? 5 * LPI : 63), 15>(); break;
            case 6: wait_cnt<(6 * LPI < 63 ? 6 * LPI : 63), 15>(); break;
            default: wait_cnt<(7 * LPI < 63 ? 7 * LPI : 63), 15>(); break;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float d = fmaf(half_to_float(sc[s][r][j]), chunk_dot(w[s][r][j], xr[j]), v);
                v = ok[j] ? d : v;
            }
            acc[r * RW + i] = v;
        }
        if (i + P < RW) issue(s, i + P);
    }

    wave_reduce<V>(acc);
    if constexpr (KS > 1 || EPI == kEpiSwiglu) {
        __shared__ float red[4][V];
        for_each_reduced<V>(acc, lane, [&](int idx, float val) { red[wave][idx] = val; });
        __syncthreads();
        if (part == 0) {
            for (int i = lane; i < n_out; i += kWave) {
                float t0 = red[wave][i];
#pragma unroll
                for (int p = 1; p < KS; ++p) t0 += red[wave + p][i];
                const int64_t o = o0 + i;
                if constexpr (EPI == kEpiSwiglu) {
                    float t1 = red[wave][RW + i];
#pragma unroll
                    for (int p = 1; p < KS; ++p) t1 += red[wave + p][RW + i];
                    a.Y[o] = silu_mul(t0, t1);
                } else {
                    a.Y[o] = EPI == kEpiAdd ? t0 + a.R[o] : t0;
                }
            }
        }
    } else {
        for_each_reduced<V>(acc, lane, [&](int idx, float val) {
            if (idx >= n_out) return;
            const int64_t o = o0 + idx;
            a.Y[o] = EPI == kEpiAdd ? val + a.R[o] : val;
        });
    }
}

// Chunks per lane a shape needs with KS slices: the candidates of one (KS, J)
// apply only where J is exactly that, so no lane carries unused x registers.
static int q4x_chunks_per_lane(int K, int KS) {
    const int C = (K / 32 + KS - 1) / KS;
    return (C + kWave - 1) / kWave;
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

// `rows` = RW weight rows per wavefront group at most (for the gated product
// the launch passes 2N rows, so a group takes up to (RW + 1) / 2 outputs, two
// rows each).  The workgroup count is rounded up to a multiple of the compute
// units, so every unit streams the same number of rows (+-1 per group).
template <int J, int KS, int RW>
static bool geom_q4x(const Variant&, int M, int N, int K, dim3* grid, size_t* lds) {
    if (M != 1 || K <= 0 || q4x_chunks_per_lane(K, KS) != J) return false;
    constexpr int64_t per_block = (int64_t)RW * (4 / KS);
    int64_t blocks = (N + per_block - 1) / per_block;
    const int cus = device_cus();
    if (cus > 0) blocks = (blocks + cus - 1) / cus * cus;
    // the resources address RW rows of codes with 32-bit offsets
    if ((int64_t)RW * (K / 2) > 0x7FFFFFFF) return false;
    *grid = dim3((unsigned)blocks);
    *lds = 0;
    return true;
}

template <int J, int KS, int P, int RW>
static void add_q4x(std::vector<Variant>& out) {
    Variant v{};
    v.kind = LIN_KIND_GEMV_Q4G64;
    v.cfg.algo = LIN_ALGO_VALU;
    v.cfg.rows = RW;
    v.cfg.unroll = P;
    v.cfg.split = KS;
    v.cfg.stage_x = 2;   // x resident in registers, rows streamed
    v.cfg.tile_m = 1;
    v.mt = 1;
    v.min_m = 1;
    v.func = (const void*)&gemv_q4_xres<J, KS, P, RW, kEpiNone>;
    v.epi[kEpiAdd] = (const void*)&gemv_q4_xres<J, KS, P, RW, kEpiAdd>;
    v.epi[kEpiSwiglu] = (const void*)&gemv_q4_xres<J, KS, P, (RW + 1) / 2, kEpiSwiglu>;
    v.geometry = &geom_q4x<J, KS, RW>;
    out.push_back(v);
}

template <int J, int KS, int P>
static void add_q4x_rows(std::vector<Variant>& out) {
    add_q4x<J, KS, P, 4>(out);
    add_q4x<J, KS, P, 7>(out);
    add_q4x<J, KS, P, 10>(out);
    add_q4x<J, KS, P, 14>(out);
    add_q4x<J, KS, P, 20>(out);
}

template <int J, int KS>
static void add_q4x_pipes(std::vector<Variant>& out) {
    add_q4x_rows<J, KS, 2>(out);
    add_q4x_rows<J, KS, 4>(out);
    if constexpr (J <= 3) {   // an 8-deep pipeline where the wait counter holds it
        add_q4x<J, KS, 8, 10>(out);
        add_q4x<J, KS, 8, 14>(out);
        add_q4x<J, KS, 8, 20>(out);
    }
}

void register_gemv_q4x(std::vector<Variant>& out) {
    add_q4x_pipes<1, 1>(out);
    add_q4x_pipes<2, 1>(out);
    add_q4x_pipes<3, 1>(out);
    add_q4x_pipes<1, 2>(out);
    add_q4x_pipes<2, 2>(out);
    add_q4x_pipes<3, 2>(out);
    add_q4x_pipes<4, 2>(out);
    add_q4x_pipes<5, 2>(out);
    add_q4x_pipes<1, 4>(out);
    add_q4x_pipes<2, 4>(out);
    add_q4x_pipes<3, 4>(out);
}

}  // namespace lin

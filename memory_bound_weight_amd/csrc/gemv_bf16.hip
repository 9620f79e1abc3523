// Standalone kernels, launch geometry and the candidate list of the product in
// gemv_bf16_impl.h.
#include "gemv_bf16_impl.h"
#include "registry.h"

namespace lin {

template <int MT, int R, int U, int SPLIT, bool STAGE, int EPI = kEpiNone, bool NORM = false>
__global__ __launch_bounds__(kBlock) void gemv_bf16_valu(KArgs a) {
    gemv_bf16_valu_block<MT, R, U, SPLIT, STAGE, EPI, NORM>(a, blockIdx.x);
}

template <int MT, int R, int U, int SPLIT, bool STAGE>
static bool geom_bf16(const Variant&, int M, int N, int K, dim3* grid, size_t* lds) {
    constexpr int rows_per_block = R * (4 / SPLIT);
    size_t bytes = STAGE ? 16 * stage_x_units(MT, K) : 0;
    if (bytes > kMaxDynLds) return false;
    (void)M;
    *grid = dim3((unsigned)((N + rows_per_block - 1) / rows_per_block));
    *lds = bytes;
    return true;
}

// The RMSNorm prologue also stages the gain next to x.
template <int MT, int R, int U, int SPLIT, bool STAGE>
static bool geom_bf16_norm(const Variant& v, int M, int N, int K, dim3* grid, size_t* lds) {
    if (!geom_bf16<MT, R, U, SPLIT, STAGE>(v, M, N, K, grid, lds)) return false;
    *lds += 16 * stage_x_units(1, K);
    return *lds <= kMaxDynLds;
}

template <int MT, int R, int U, int SPLIT, bool STAGE>
static void add(std::vector<Variant>& out) {
    // The gated form keeps R weight rows per wavefront: R/2 gate rows and the
    // matching up rows (one of each for R = 1).
    constexpr int RS = R >= 2 ? R / 2 : 1;
    Variant v{};
    v.cfg.algo = LIN_ALGO_VALU;
    v.cfg.rows = R;
    v.cfg.unroll = U;
    v.cfg.split = SPLIT;
    v.cfg.stage_x = STAGE ? 1 : 0;
    v.cfg.tile_m = MT;
    v.mt = MT;
    v.min_m = MT / 2 + 1;
    v.func = (const void*)&gemv_bf16_valu<MT, R, U, SPLIT, STAGE>;
    v.geometry = &geom_bf16<MT, R, U, SPLIT, STAGE>;
    if (MT <= LIN_GEMV_MAX_M) {
        v.kind = LIN_KIND_GEMV_BF16;
        if constexpr (MT <= LIN_GEMV_MAX_M) {
            v.epi[kEpiAdd] = (const void*)&gemv_bf16_valu<MT, R, U, SPLIT, STAGE, kEpiAdd>;
            v.epi[kEpiSwiglu] = (const void*)&gemv_bf16_valu<MT, RS, U, SPLIT, STAGE, kEpiSwiglu>;
            if constexpr (STAGE && MT == 1) {
                Variant n = v;
                n.kind = LIN_KIND_GEMV_BF16_NORM;
                n.func = (const void*)&gemv_bf16_valu<MT, R, U, SPLIT, STAGE, kEpiNone, true>;
                n.epi[kEpiAdd] = (const void*)&gemv_bf16_valu<MT, R, U, SPLIT, STAGE, kEpiAdd, true>;
                n.epi[kEpiSwiglu] = (const void*)&gemv_bf16_valu<MT, RS, U, SPLIT, STAGE, kEpiSwiglu, true>;
                n.geometry = &geom_bf16_norm<MT, R, U, SPLIT, STAGE>;
                out.push_back(n);
            }
        }
        out.push_back(v);
        v.epi[kEpiAdd] = v.epi[kEpiSwiglu] = nullptr;
    }
    v.kind = LIN_KIND_SKINNY_BF16;
    out.push_back(v);
}

template <int MT, int R, int U>
static void add_splits(std::vector<Variant>& out) {
    add<MT, R, U, 1, false>(out);
    add<MT, R, U, 2, false>(out);
    add<MT, R, U, 4, false>(out);
    add<MT, R, U, 1, true>(out);
    add<MT, R, U, 2, true>(out);
    add<MT, R, U, 4, true>(out);
}

void register_gemv_bf16(std::vector<Variant>& out) {
    add_splits<1, 1, 2>(out);
    add_splits<1, 1, 4>(out);
    add_splits<1, 2, 1>(out);
    add_splits<1, 2, 2>(out);
    add_splits<1, 2, 4>(out);
    add_splits<1, 4, 1>(out);
    add_splits<1, 4, 2>(out);
    add_splits<1, 8, 1>(out);
    // K = 3584 has 448 chunks, 7 x 64: one wavefront per row with seven loads
    // per lane covers it with no idle lanes (every split leaves some idle)
    add<1, 1, 7, 1, false>(out);
    add<1, 1, 7, 1, true>(out);
    add<1, 2, 7, 1, false>(out);
    add<1, 2, 7, 1, true>(out);

    add_splits<2, 1, 2>(out);
    add_splits<2, 2, 1>(out);
    add_splits<2, 2, 2>(out);
    add_splits<2, 4, 1>(out);

    add_splits<4, 1, 2>(out);
    add_splits<4, 2, 1>(out);
    add_splits<4, 2, 2>(out);
    add_splits<4, 4, 1>(out);

    add_splits<8, 1, 1>(out);
    add_splits<8, 1, 2>(out);
    add_splits<8, 2, 1>(out);
    add_splits<8, 4, 1>(out);
    add_splits<8, 2, 2>(out);
    add_splits<8, 4, 2>(out);
    add_splits<8, 8, 1>(out);

    add_splits<16, 1, 1>(out);
    add_splits<16, 2, 1>(out);

    add_splits<32, 1, 1>(out);
}

}  // namespace lin

// Standalone kernels, launch geometry and candidates of the vector-ALU int4
// product over the tiled layout (gemv_q4t_impl.h): the M <= 8 candidates of
// LIN_KIND_SKINNY_Q4G64 for M <= 2.  `rows` counts 16-row tiles per wavefront,
// `unroll` the 128-k blocks per pipeline stage.
#include "gemv_q4t_impl.h"
#include "registry.h"

namespace lin {

template <int MT, int R, int U, int SPLIT>
__global__ __launch_bounds__(kBlock) void gemv_q4t_valu(KArgs a) {
    gemv_q4t_valu_block<MT, R, U, SPLIT>(a, blockIdx.x);
}

template <int MT, int R, int U, int SPLIT>
static bool geom_q4t(const Variant&, int M, int N, int K, dim3* grid, size_t* lds) {
    (void)M;
    (void)K;
    const int tiles = (N + 15) / 16;
    constexpr int per_block = R * (4 / SPLIT);
    *grid = dim3((unsigned)((tiles + per_block - 1) / per_block));
    *lds = 0;
    return true;
}

template <int MT, int R, int U, int SPLIT>
static void add(std::vector<Variant>& out) {
    Variant v{};
    v.kind = LIN_KIND_SKINNY_Q4G64;
    v.cfg.algo = LIN_ALGO_VALU;
    v.cfg.rows = R;
    v.cfg.unroll = U;
    v.cfg.split = SPLIT;
    v.cfg.stage_x = 0;
    v.cfg.tile_m = MT;
    v.mt = MT;
    v.min_m = MT / 2 + 1;
    v.func = (const void*)&gemv_q4t_valu<MT, R, U, SPLIT>;
    v.geometry = &geom_q4t<MT, R, U, SPLIT>;
    out.push_back(v);
}

template <int MT, int R, int U>
static void add_splits(std::vector<Variant>& out) {
    add<MT, R, U, 1>(out);
    add<MT, R, U, 2>(out);
    add<MT, R, U, 4>(out);
}

void register_gemv_q4t(std::vector<Variant>& out) {
    add_splits<1, 1, 2>(out);
    add_splits<1, 1, 4>(out);
    add_splits<1, 2, 2>(out);
    add_splits<2, 1, 2>(out);
    add_splits<2, 1, 4>(out);
    add_splits<2, 2, 2>(out);
    // M = 3 .. 8: the per-lane x of four or eight tokens leaves too few bytes
    // in flight; the matrix-core kernel is faster there (measured), so no
    // candidates are offered.
}

}  // namespace lin

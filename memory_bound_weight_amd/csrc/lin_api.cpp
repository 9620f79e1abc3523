// C-ABI layer of the linear-layer library: argument checks, the per-device
// configuration table, load-time tuning and kernel launches.  No entry point
// that computes a product allocates or synchronises.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/lin.h"
#include "registry.h"

namespace lin {
namespace {

const std::vector<Variant>& registry() {
    static std::vector<Variant>* reg = [] {
        auto* r = new std::vector<Variant>();
        register_gemv_bf16(*r);
        register_gemv_q4g64(*r);
        register_gemm_mfma(*r);
        register_gemm_mfma_ring(*r);
        register_gemm_q4_ring(*r);
        register_gemv_i8(*r);
        register_gemv_q4t(*r);
        register_gemv_q4x(*r);
        return r;
    }();
    return *reg;
}

bool valid_kind(int kind) { return kind >= LIN_KIND_GEMV_BF16 && kind <= LIN_KIND_GEMV_I8_NORM; }
bool norm_kind(int kind) {
    return kind == LIN_KIND_GEMV_BF16_NORM || kind == LIN_KIND_GEMV_Q4G64_NORM ||
           kind == LIN_KIND_GEMV_I8_NORM;
}

using Key = std::tuple<int, int, int64_t, int64_t, int64_t>;   // device, kind, M, N, K

std::mutex g_mu;
std::map<Key, int>& table() {   // value: index into registry()
    static auto* t = new std::map<Key, int>();
    return *t;
}

int pow2ceil(int64_t m) {
    int p = 1;
    while (p < m) p <<= 1;
    return p;
}

bool same_cfg(const lin_config& a, const lin_config& b) {
    return a.algo == b.algo && a.rows == b.rows && a.unroll == b.unroll && a.split == b.split &&
           a.stage_x == b.stage_x && a.tile_m == b.tile_m && a.waves == b.waves;
}

bool applicable(const Variant& v, int kind, int64_t M, int64_t N, int64_t K) {
    if (v.kind != kind) return false;
    if (v.cfg.algo == LIN_ALGO_VALU) {
        if (v.mt != pow2ceil(M)) return false;
    } else {
        if (M < v.min_m || (K == 0 && kind != LIN_KIND_SKINNY_Q4G64)) return false;
    }
    dim3 g;
    size_t lds;
    return v.geometry(v, (int)M, (int)N, (int)K, &g, &lds);
}

std::vector<int> candidates(int kind, int64_t M, int64_t N, int64_t K) {
    std::vector<int> out;
    const auto& reg = registry();
    for (int i = 0; i < (int)reg.size(); ++i)
        if (applicable(reg[i], kind, M, N, K)) out.push_back(i);
    return out;
}

int find_variant(int kind, int64_t M, int64_t N, int64_t K, const lin_config& cfg) {
    for (int i : candidates(kind, M, N, K))
        if (same_cfg(registry()[i].cfg, cfg)) return i;
    return -1;
}

size_t workspace_need(const Variant& v, int64_t M, int64_t N, int64_t K);

// Built-in choice for shapes that were neither tuned nor pinned.
int default_variant(int kind, int64_t M, int64_t N, int64_t K) {
    lin_config want{};
    want.algo = LIN_ALGO_VALU;
    want.tile_m = pow2ceil(M);
    const int mt = want.tile_m;
    if (kind == LIN_KIND_SKINNY_Q4G64) {
        // matrix cores without split-K: the token tile that covers M best
        const int tm = mt <= 16 ? 16 : (mt <= 32 ? 32 : (mt <= 64 ? 64 : 128));
        for (int i : candidates(kind, M, N, K)) {
            const Variant& v = registry()[i];
            if (v.cfg.split == 1 && v.cfg.tile_m == tm && v.cfg.rows == 128) return i;
        }
        for (int i : candidates(kind, M, N, K))
            if (workspace_need(registry()[i], M, N, K) == 0) return i;
        return -1;
    }
    if (norm_kind(kind)) {
        // every workgroup repeats the prologue: several rows per workgroup
        want.rows = N >= 4096 ? 4 : 2;
        want.unroll = kind == LIN_KIND_GEMV_BF16_NORM ? 2 : 1;
        want.split = N >= 4096 ? 1 : 2;
        want.stage_x = 1;
        int i = find_variant(kind, M, N, K, want);
        if (i >= 0) return i;
        auto c = candidates(kind, M, N, K);
        return c.empty() ? -1 : c.front();
    }
    if (kind == LIN_KIND_GEMV_I8) {
        want.rows = 2;
        want.unroll = mt <= 1 ? 2 : 1;
        want.split = N >= 4096 ? 1 : (N >= 1024 ? 2 : 4);
    } else if (kind == LIN_KIND_GEMV_Q4G64) {
        want.rows = mt <= 1 ? 4 : (mt <= 4 ? 2 : 1);
        want.unroll = 1;
        want.split = N >= 4096 ? 1 : (N >= 1024 ? 2 : 4);
    } else {
        if (kind == LIN_KIND_SKINNY_BF16 && M > 16) {
            // matrix cores without split-K (the default never needs the
            // workspace): the LDS-ring variant whose token tile covers M best
            const int tm = mt < 32 ? 32 : (mt > 256 ? 256 : mt);
            const int bn = tm == 32 ? 32 : (tm == 256 ? 128 : 64);
            const int tm_pick = tm == 256 ? 128 : tm;
            for (int i : candidates(kind, M, N, K)) {
                const Variant& v = registry()[i];
                if (v.cfg.algo != LIN_ALGO_MFMA || v.cfg.stage_x != 4 || v.cfg.split != 1 ||
                    v.cfg.waves != 0)
                    continue;
                if (v.cfg.tile_m == tm_pick && v.cfg.rows == bn) return i;
            }
            for (int i : candidates(kind, M, N, K))
                if (registry()[i].cfg.algo == LIN_ALGO_MFMA && workspace_need(registry()[i], M, N, K) == 0)
                    return i;
        }
        want.rows = mt <= 1 ? (N >= 8192 ? 2 : 1) : (mt <= 8 ? 2 : 1);
        want.unroll = mt <= 1 ? (want.rows == 1 ? 4 : 2) : (mt <= 8 ? 2 : 1);
        if (mt == 4 || mt == 8) want.rows = 2, want.unroll = 2;
        if (mt >= 16) want.rows = 1, want.unroll = (mt == 16 ? 2 : 1);
        want.split = N >= 8192 ? 1 : (N >= 2048 ? 2 : 4);
    }
    want.stage_x = 0;
    int i = find_variant(kind, M, N, K, want);
    if (i >= 0) return i;
    auto c = candidates(kind, M, N, K);
    return c.empty() ? -1 : c.front();
}

int current_device() {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) return -1;
    return d;
}

std::map<Key, int>& default_cache() {   // built-in choices already worked out
    static auto* t = new std::map<Key, int>();
    return *t;
}

// Variant for the next call: tuned or pinned entry, else the (cached) default.
int lookup(int kind, int64_t M, int64_t N, int64_t K) {
    const int dev = current_device();
    const Key key(dev, kind, M, N, K);
    const Key dkey(0, kind, M, N, K);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = table().find(key);
        if (it != table().end()) return it->second;
        auto dt = default_cache().find(dkey);
        if (dt != default_cache().end()) return dt->second;
    }
    const int vi = default_variant(kind, M, N, K);
    std::lock_guard<std::mutex> lk(g_mu);
    default_cache()[dkey] = vi;
    return vi;
}

// Split-K workspace per device.  Grown only by the load-time calls
// (lin_autotune, lin_set_config), after a device synchronisation, and zeroed so
// that every tile counter starts at 0; kernels leave the counters at 0.  A
// launch bakes the workspace address into its arguments, and a graph captured
// from it keeps that address, so a workspace is never freed: when it grows,
// the old buffer stays allocated (and its counters at 0) until the process
// ends, and graphs captured before the growth keep working on it.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    std::vector<void*> retired;   // earlier, smaller buffers (never freed)
};
std::map<int, Workspace>& workspaces() {
    static auto* w = new std::map<int, Workspace>();
    return *w;
}

size_t workspace_need(const Variant& v, int64_t M, int64_t N, int64_t K) {
    return v.workspace ? v.workspace(v, (int)M, (int)N, (int)K) : 0;
}

int ensure_workspace(int dev, size_t bytes) {
    if (bytes == 0) return LIN_OK;
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& w = workspaces()[dev];
    if (w.bytes >= bytes) return LIN_OK;
    if (hipDeviceSynchronize() != hipSuccess) return LIN_ERR_HIP;
    const size_t want = bytes + (bytes >> 2);   // headroom for nearby shapes
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) return LIN_ERR_HIP;
    if (hipMemset(p, 0, want) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        w.retired.push_back(p);   // not handed out; kept like the others
        return LIN_ERR_HIP;
    }
    if (w.ptr) w.retired.push_back(w.ptr);
    w.ptr = p;
    w.bytes = want;
    return LIN_OK;
}

// Dynamic LDS above the default 64 KB per workgroup must be allowed per
// kernel and device first; the largest size allowed so far is kept per
// (device, kernel).
bool allow_lds(size_t lds, const void* func) {
    if (lds <= 64 * 1024) return true;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    static auto* allowed = new std::map<std::pair<int, const void*>, size_t>();
    std::lock_guard<std::mutex> lk(g_mu);
    auto ins = allowed->emplace(std::make_pair(dev, func), (size_t)64 * 1024);
    size_t& cur = ins.first->second;
    if (lds <= cur) return true;
    if (hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return false;
    cur = lds;
    return true;
}

// geom_n: the row count the launch grid is sized for, when it differs from a.N
// (the gated epilogue).
// ws: split-K workspace to use instead of the device's library-owned one
// (the static scratch of the allocation-free entry point), or nullptr.
int launch_variant(int vi, const KArgs& a, hipStream_t stream, hipEvent_t ev0 = nullptr,
                   hipEvent_t ev1 = nullptr, const void* func = nullptr, int64_t geom_n = -1,
                   void* ws = nullptr) {
    const Variant& v = registry()[vi];
    if (!func) func = v.func;
    dim3 grid;
    size_t lds = 0;
    if (!v.geometry(v, a.M, geom_n >= 0 ? (int)geom_n : a.N, a.K, &grid, &lds))
        return LIN_ERR_UNSUPPORTED;
    if (!allow_lds(lds, func)) return LIN_ERR_HIP;
    KArgs args = a;
    args.splits = v.cfg.algo == LIN_ALGO_MFMA ? v.cfg.split : 1;
    args.ws = nullptr;
    const size_t need = workspace_need(v, a.M, a.N, a.K);
    if (need && ws) {
        args.ws = ws;
    } else if (need) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return LIN_ERR_HIP;
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = workspaces().find(dev);
        if (it == workspaces().end() || it->second.bytes < need) return LIN_ERR_UNSUPPORTED;
        args.ws = it->second.ptr;
    }
    void* params[] = {(void*)&args};
    const dim3 block(v.block ? v.block : kBlock);
    hipError_t e;
    if (ev0 || ev1)
        e = hipExtLaunchKernel(func, grid, block, params, lds, stream, ev0, ev1, 0);
    else
        e = hipLaunchKernel(func, grid, block, params, lds, stream);
    return e == hipSuccess ? LIN_OK : LIN_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Grid rows of a gated-epilogue launch with N outputs: a wavefront of a
// configuration with `rows` >= 2 weight rows takes rows/2 outputs (gate and up
// rows), so the grid is sized as for 2N rows; with rows == 1 it takes one
// output (two weight rows), as for N rows.
int64_t swiglu_grid_rows(const Variant& v, int64_t N) { return v.cfg.rows >= 2 ? 2 * N : N; }



// Shared argument checks.  Returns LIN_OK, a negative status, or 1 for an
// empty call (nothing to do).
int check(int kind, const void* W, const void* S, const void* x, const float* y, int64_t M,
          int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return LIN_ERR_SHAPE;
    const bool q4 = kind == LIN_KIND_GEMV_Q4G64 || kind == LIN_KIND_SKINNY_Q4G64 ||
                    kind == LIN_KIND_GEMV_Q4G64_NORM;
    const bool i8 = kind == LIN_KIND_GEMV_I8 || kind == LIN_KIND_GEMV_I8_NORM;
    const int64_t maxm = (kind == LIN_KIND_SKINNY_BF16 || kind == LIN_KIND_SKINNY_Q4G64)
                             ? LIN_SKINNY_MAX_M
                             : (norm_kind(kind) ? 1 : LIN_GEMV_MAX_M);
    if (M > maxm || N > 0x7FFFFFFF || K > LIN_MAX_K) return LIN_ERR_SHAPE;
    if (q4 ? (K % 64) : (i8 ? (K % 16) : (K % 8))) return LIN_ERR_SHAPE;
    if (M == 0 || N == 0) return 1;
    if (norm_kind(kind) && K == 0) return LIN_ERR_SHAPE;   // the mean square needs K >= 1
    if (!y) return LIN_ERR_NULL;
    if (K > 0 && (!W || !x || ((q4 || i8) && !S))) return LIN_ERR_NULL;
    if (!aligned(y, 4)) return LIN_ERR_ALIGN;
    if (K > 0) {
        if (!aligned(W, 16) || !aligned(x, 16)) return LIN_ERR_ALIGN;
        if ((kind == LIN_KIND_GEMV_Q4G64 || kind == LIN_KIND_GEMV_Q4G64_NORM) && !aligned(S, 2))
            return LIN_ERR_ALIGN;
        if (kind == LIN_KIND_SKINNY_Q4G64 && !aligned(S, 16)) return LIN_ERR_ALIGN;
        if (i8 && !aligned(S, 4)) return LIN_ERR_ALIGN;
    }
    return LIN_OK;
}

int run(int kind, const void* W, const void* S, const void* x, float* y, int64_t M, int64_t N,
        int64_t K, void* stream) {
    int st = check(kind, W, S, x, y, M, N, K);
    if (st != LIN_OK) return st > 0 ? LIN_OK : st;
    const int vi = lookup(kind, M, N, K);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    KArgs a{W, S, x, y, (int)M, (int)N, (int)K, 1, nullptr};
    return launch_variant(vi, a, (hipStream_t)stream);
}

struct Flush {
    void* buf = nullptr;
    size_t bytes = 0;
};
std::map<int, Flush>& flushes() {
    static auto* f = new std::map<int, Flush>();
    return *f;
}

}  // namespace
}  // namespace lin

using namespace lin;

extern "C" {

int lin_version(void) { return (1 << 16) | 0; }

const char* lin_status_string(int status) {
    switch (status) {
        case LIN_OK: return "ok";
        case LIN_ERR_NULL: return "a required pointer is NULL";
        case LIN_ERR_SHAPE: return "M, N or K out of range for this product";
        case LIN_ERR_ALIGN: return "a pointer is not aligned as the product requires";
        case LIN_ERR_UNSUPPORTED: return "configuration not available for this shape";
        case LIN_ERR_HIP: return "the HIP runtime reported an error";
        case LIN_ERR_ARG: return "invalid argument";
        case LIN_ERR_SCRATCH:
            return "the product needs more split-K scratch than the static array holds "
                   "(LIN_STATIC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int lin_gemv_bf16(const void* W, const void* x, float* y, int64_t M, int64_t N, int64_t K,
                  void* stream) {
    return run(LIN_KIND_GEMV_BF16, W, nullptr, x, y, M, N, K, stream);
}

int lin_gemv_q4g64(const void* Wq, const void* S, const void* x, float* y, int64_t M, int64_t N,
                   int64_t K, void* stream) {
    return run(LIN_KIND_GEMV_Q4G64, Wq, S, x, y, M, N, K, stream);
}

int lin_gemm_skinny_bf16(const void* W, const void* X, float* Y, int64_t M, int64_t N, int64_t K,
                         void* stream) {
    return run(LIN_KIND_SKINNY_BF16, W, nullptr, X, Y, M, N, K, stream);
}

// Product of up to LIN_GEMV_MAX_M tokens with a fused epilogue, in the
// configuration tuned or pinned for the plain product of the same weight
// matrix (2N rows for the gated one).
static int run_epilogue(int kind, const void* W, const void* S, const void* x, float* y,
                        int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                        void* stream) {
    if (epilogue < LIN_EPI_NONE || epilogue > LIN_EPI_SWIGLU) return LIN_ERR_ARG;
    if (N < 0 || N > 0x3FFFFFFF) return LIN_ERR_SHAPE;
    const int64_t NW = epilogue == LIN_EPI_SWIGLU ? 2 * N : N;   // weight rows
    int st = check(kind, W, S, x, y, M, NW, K);   // 1 <= M <= LIN_GEMV_MAX_M
    if (st != LIN_OK) return st > 0 ? LIN_OK : st;
    if (epilogue == LIN_EPI_ADD) {
        if (!r) return LIN_ERR_NULL;
        if (!aligned(r, 4)) return LIN_ERR_ALIGN;
    }
    const int vi = lookup(kind, M, NW, K);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    const Variant& v = registry()[vi];
    const void* f = epilogue == LIN_EPI_NONE ? v.func : v.epi[epilogue];
    if (!f) return LIN_ERR_UNSUPPORTED;
    KArgs a{W, S, x, y, (int)M, (int)N, (int)K, 1, nullptr, r};
    return launch_variant(vi, a, (hipStream_t)stream, nullptr, nullptr, f,
                          epilogue == LIN_EPI_SWIGLU ? swiglu_grid_rows(v, N) : -1);
}

int lin_gemv_bf16_ep(const void* W, const void* x, float* y, int64_t M, int64_t N, int64_t K,
                     int epilogue, const float* r, void* stream) {
    return run_epilogue(LIN_KIND_GEMV_BF16, W, nullptr, x, y, M, N, K, epilogue, r, stream);
}

int lin_gemv_q4g64_ep(const void* Wq, const void* S, const void* x, float* y, int64_t M,
                      int64_t N, int64_t K, int epilogue, const float* r, void* stream) {
    return run_epilogue(LIN_KIND_GEMV_Q4G64, Wq, S, x, y, M, N, K, epilogue, r, stream);
}

// Batch-1 product of RMSNorm(x) with an optional epilogue, in the configuration
// tuned or pinned for the matrix under the prologue kind.
static int run_norm(int kind, const void* W, const void* S, const void* x, const void* g,
                    float eps, float* y, int64_t M, int64_t N, int64_t K, int epilogue,
                    const float* r, void* stream) {
    if (epilogue < LIN_EPI_NONE || epilogue > LIN_EPI_SWIGLU) return LIN_ERR_ARG;
    if (!(eps >= 0.f) || eps > 3.0e38f) return LIN_ERR_ARG;   // also rejects NaN
    if (N < 0 || N > 0x3FFFFFFF) return LIN_ERR_SHAPE;
    if (M != 0 && M != 1) return LIN_ERR_SHAPE;
    const int64_t NW = epilogue == LIN_EPI_SWIGLU ? 2 * N : N;   // weight rows
    int st = check(kind, W, S, x, y, M, NW, K);
    if (st != LIN_OK) return st > 0 ? LIN_OK : st;
    if (!g) return LIN_ERR_NULL;
    if (!aligned(g, 16)) return LIN_ERR_ALIGN;
    if (epilogue == LIN_EPI_ADD) {
        if (!r) return LIN_ERR_NULL;
        if (!aligned(r, 4)) return LIN_ERR_ALIGN;
    }
    const int vi = lookup(kind, M, NW, K);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    const Variant& v = registry()[vi];
    const void* f = epilogue == LIN_EPI_NONE ? v.func : v.epi[epilogue];
    if (!f) return LIN_ERR_UNSUPPORTED;
    KArgs a{W, S, x, y, (int)M, (int)N, (int)K, 1, nullptr, r, g, eps};
    return launch_variant(vi, a, (hipStream_t)stream, nullptr, nullptr, f,
                          epilogue == LIN_EPI_SWIGLU ? swiglu_grid_rows(v, N) : -1);
}

int lin_gemv_bf16_norm(const void* W, const void* x, const void* g, float eps, float* y,
                       int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                       void* stream) {
    return run_norm(LIN_KIND_GEMV_BF16_NORM, W, nullptr, x, g, eps, y, M, N, K, epilogue, r,
                    stream);
}

int lin_gemv_q4g64_norm(const void* Wq, const void* S, const void* x, const void* g, float eps,
                        float* y, int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                        void* stream) {
    return run_norm(LIN_KIND_GEMV_Q4G64_NORM, Wq, S, x, g, eps, y, M, N, K, epilogue, r,
                    stream);
}

int lin_gemv_i8(const void* Wq, const void* S, const void* x, float* y, int64_t M, int64_t N,
                int64_t K, void* stream) {
    return run(LIN_KIND_GEMV_I8, Wq, S, x, y, M, N, K, stream);
}

int lin_gemv_i8_ep(const void* Wq, const void* S, const void* x, float* y, int64_t M, int64_t N,
                   int64_t K, int epilogue, const float* r, void* stream) {
    return run_epilogue(LIN_KIND_GEMV_I8, Wq, S, x, y, M, N, K, epilogue, r, stream);
}

int lin_gemv_i8_norm(const void* Wq, const void* S, const void* x, const void* g, float eps,
                     float* y, int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                     void* stream) {
    return run_norm(LIN_KIND_GEMV_I8_NORM, Wq, S, x, g, eps, y, M, N, K, epilogue, r, stream);
}

int lin_gemm_skinny_q4g64(const void* Wt, const void* St, const void* X, float* Y, int64_t M,
                          int64_t N, int64_t K, void* stream) {
    return run(LIN_KIND_SKINNY_Q4G64, Wt, St, X, Y, M, N, K, stream);
}

int lin_q4g64_tiled_size(int64_t N, int64_t K, int64_t* wt_bytes, int64_t* st_bytes) {
    if (N < 0 || K < 0 || N > 0x7FFFFFFF || K > LIN_MAX_K || K % 64) return LIN_ERR_SHAPE;
    if (!wt_bytes || !st_bytes) return LIN_ERR_NULL;
    q4g64_tiled_bytes(N, K, wt_bytes, st_bytes);
    return LIN_OK;
}

int lin_q4g64_tile(const void* Wq, const void* S, void* Wt, void* St, int64_t N, int64_t K,
                   void* stream) {
    if (N < 0 || K < 0 || N > 0x7FFFFFFF || K > LIN_MAX_K || K % 64) return LIN_ERR_SHAPE;
    if (N == 0 || K == 0) return LIN_OK;
    if (!Wq || !S || !Wt || !St) return LIN_ERR_NULL;
    if (!aligned(Wq, 16) || !aligned(S, 2) || !aligned(Wt, 16) || !aligned(St, 16))
        return LIN_ERR_ALIGN;
    hipError_t e = launch_tile_q4g64(Wq, S, Wt, St, (int)N, (int)K, (hipStream_t)stream);
    return e == hipSuccess ? LIN_OK : LIN_ERR_HIP;
}

int lin_num_candidates(int kind, int64_t M, int64_t N, int64_t K) {
    if (!valid_kind(kind)) return LIN_ERR_ARG;
    int st = check(kind, (void*)16, (void*)16, (void*)16, (float*)16, M, N, K);
    if (st < 0) return st;
    if (st > 0) return 0;
    return (int)candidates(kind, M, N, K).size();
}

int lin_candidate(int kind, int64_t M, int64_t N, int64_t K, int index, lin_config* out) {
    if (!out) return LIN_ERR_NULL;
    int n = lin_num_candidates(kind, M, N, K);
    if (n < 0) return n;
    if (index < 0 || index >= n) return LIN_ERR_ARG;
    *out = registry()[candidates(kind, M, N, K)[index]].cfg;
    out->us = 0.f;
    return LIN_OK;
}

int lin_get_config(int kind, int64_t M, int64_t N, int64_t K, lin_config* out) {
    if (!out) return LIN_ERR_NULL;
    int n = lin_num_candidates(kind, M, N, K);
    if (n < 0) return n;
    if (n == 0) return LIN_ERR_UNSUPPORTED;
    const int vi = lookup(kind, M, N, K);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    *out = registry()[vi].cfg;
    out->us = 0.f;
    return LIN_OK;
}

static int set_config_table(int kind, int64_t M, int64_t N, int64_t K, const lin_config* cfg) {
    int n = lin_num_candidates(kind, M, N, K);
    if (n < 0) return n;
    const int dev = current_device();
    if (dev < 0) return LIN_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!cfg) {
        table().erase(Key(dev, kind, M, N, K));
        return LIN_OK;
    }
    const int vi = find_variant(kind, M, N, K, *cfg);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    table()[Key(dev, kind, M, N, K)] = vi;
    return LIN_OK;
}

}  // extern "C"

namespace lin {
namespace {
int set_config_reserving(int kind, int64_t M, int64_t N, int64_t K, const lin_config* cfg) {
    if (cfg) {
        int n = lin_num_candidates(kind, M, N, K);
        if (n < 0) return n;
        const int vi = find_variant(kind, M, N, K, *cfg);
        if (vi < 0) return LIN_ERR_UNSUPPORTED;
        const int dev = current_device();
        if (dev < 0) return LIN_ERR_HIP;
        int rc = ensure_workspace(dev, workspace_need(registry()[vi], M, N, K));
        if (rc != LIN_OK) return rc;
        // enable the dynamic LDS the configuration needs now, not at its
        // first launch (which may be inside a graph capture)
        dim3 grid;
        size_t lds = 0;
        const Variant& v = registry()[vi];
        if (v.geometry(v, (int)M, (int)N, (int)K, &grid, &lds)) {
            for (const void* f : {v.func, v.epi[kEpiAdd], v.epi[kEpiSwiglu]})
                if (f && !allow_lds(lds, f)) return LIN_ERR_HIP;
        }
    }
    return LIN_OK;
}
}  // namespace
}  // namespace lin

extern "C" {

int lin_set_config(int kind, int64_t M, int64_t N, int64_t K, const lin_config* cfg) {
    int rc = set_config_reserving(kind, M, N, K, cfg);
    if (rc != LIN_OK) return rc;
    return set_config_table(kind, M, N, K, cfg);
}

int lin_stream_read(const void* buf, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return LIN_ERR_SHAPE;
    if (bytes == 0) return LIN_OK;
    if (!buf) return LIN_ERR_NULL;
    if (!aligned(buf, 16)) return LIN_ERR_ALIGN;
    hipError_t e = launch_stream_read(buf, (size_t)bytes, (hipStream_t)stream);
    return e == hipSuccess ? LIN_OK : LIN_ERR_HIP;
}

int lin_quantize_q4g64(const void* W, void* Wq, void* S, int64_t N, int64_t K, void* stream) {
    if (N < 0 || K < 0 || N > 0x7FFFFFFF || K > LIN_MAX_K || K % 64) return LIN_ERR_SHAPE;
    if (N == 0 || K == 0) return LIN_OK;
    if (!W || !Wq || !S) return LIN_ERR_NULL;
    if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(S, 2)) return LIN_ERR_ALIGN;
    hipError_t e = launch_quantize_q4g64(W, Wq, S, (int)N, (int)K, (hipStream_t)stream);
    return e == hipSuccess ? LIN_OK : LIN_ERR_HIP;
}

int lin_quantize_i8(const void* W, void* Wq, void* S, int64_t N, int64_t K, void* stream) {
    if (N < 0 || K < 0 || N > 0x7FFFFFFF || K > LIN_MAX_K || K % 16) return LIN_ERR_SHAPE;
    if (N == 0 || K == 0) return LIN_OK;
    if (!W || !Wq || !S) return LIN_ERR_NULL;
    if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(S, 4)) return LIN_ERR_ALIGN;
    hipError_t e = launch_quantize_i8(W, Wq, S, (int)N, (int)K, (hipStream_t)stream);
    return e == hipSuccess ? LIN_OK : LIN_ERR_HIP;
}

int lin_autotune(int kind, const void* W, const void* S, const void* x, float* y, int64_t M,
                 int64_t N, int64_t K, void* stream, lin_config* out) {
    if (!valid_kind(kind)) return LIN_ERR_ARG;
    int st = check(kind, W, S, x, y, M, N, K);
    if (st < 0) return st;
    if (st > 0) return LIN_OK;
    const auto cand = candidates(kind, M, N, K);
    if (cand.empty()) return LIN_ERR_UNSUPPORTED;
    const int dev = current_device();
    if (dev < 0) return LIN_ERR_HIP;
    hipStream_t s = (hipStream_t)stream;

    // A buffer larger than the last-level caches (4 MB L2 per XCD, 256 MB
    // Infinity Cache); writing it before each timed call evicts the weights.
    const size_t flush_bytes = (size_t)512 << 20;
    Flush* fl;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        fl = &flushes()[dev];
        if (!fl->buf) {
            if (hipMalloc(&fl->buf, flush_bytes) != hipSuccess) {
                fl->buf = nullptr;
                return LIN_ERR_HIP;
            }
            fl->bytes = flush_bytes;
        }
    }
    size_t ws_max = 0;
    for (int vi : cand) ws_max = std::max(ws_max, workspace_need(registry()[vi], M, N, K));
    if (int rc0 = ensure_workspace(dev, ws_max)) return rc0;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return LIN_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return LIN_ERR_HIP;
    }
    // the RMSNorm kinds time the prologue with x standing in for the gain
    KArgs a{W, S, x, y, (int)M, (int)N, (int)K, 1, nullptr, nullptr, x, 1e-6f};
    const int reps = 7;
    int best = -1;
    float best_us = 0.f;
    int rc = LIN_OK;
    uint32_t salt = 1;
    for (int vi : cand) {
        std::vector<float> t;
        if ((rc = launch_variant(vi, a, s)) != LIN_OK) break;   // warm-up (code load)
        for (int r = 0; r < reps && rc == LIN_OK; ++r) {
            if (launch_flush(fl->buf, fl->bytes / 16, salt++, s) != hipSuccess) {
                rc = LIN_ERR_HIP;
                break;
            }
            if ((rc = launch_variant(vi, a, s, e0, e1)) != LIN_OK) break;
            if (hipEventSynchronize(e1) != hipSuccess) {
                rc = LIN_ERR_HIP;
                break;
            }
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
                rc = LIN_ERR_HIP;
                break;
            }
            t.push_back(ms * 1000.f);
        }
        if (rc != LIN_OK) break;
        std::sort(t.begin(), t.end());
        const float med = t[t.size() / 2];
        if (best < 0 || med < best_us) {
            best = vi;
            best_us = med;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc != LIN_OK) return rc;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        table()[Key(dev, kind, M, N, K)] = best;
    }
    if (out) {
        *out = registry()[best].cfg;
        out->us = best_us;
    }
    return LIN_OK;
}

int lin_autotune_set(int kind, const void* const* W, const void* const* S, int count,
                     const void* x, float* y, int64_t M, int64_t N, int64_t K, void* stream,
                     lin_config* out) {
    if (!valid_kind(kind)) return LIN_ERR_ARG;
    if (count < 1) return LIN_ERR_ARG;
    if (!W || ((kind == LIN_KIND_GEMV_Q4G64 || kind == LIN_KIND_SKINNY_Q4G64 ||
                kind == LIN_KIND_GEMV_I8 || kind == LIN_KIND_GEMV_Q4G64_NORM ||
                kind == LIN_KIND_GEMV_I8_NORM) && !S))
        return LIN_ERR_NULL;
    for (int j = 0; j < count; ++j) {
        const int st = check(kind, W[j], S ? S[j] : nullptr, x, y, M, N, K);
        if (st < 0) return st;
        if (st > 0) return LIN_OK;
    }
    const auto cand = candidates(kind, M, N, K);
    if (cand.empty()) return LIN_ERR_UNSUPPORTED;
    const int dev = current_device();
    if (dev < 0) return LIN_ERR_HIP;
    size_t ws_max = 0;
    for (int vi : cand) ws_max = std::max(ws_max, workspace_need(registry()[vi], M, N, K));
    if (int rc0 = ensure_workspace(dev, ws_max)) return rc0;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LIN_ERR_HIP;

    // Candidates run on a private stream (default priority), captured as one
    // graph of n launches cycling over the matrices, as a decode step runs them.
    hipStream_t ts = nullptr;
    if (hipStreamCreateWithFlags(&ts, hipStreamNonBlocking) != hipSuccess) return LIN_ERR_HIP;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = LIN_OK;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = LIN_ERR_HIP;
    const int n = count * std::max(1, (32 + count - 1) / count);
    const int reps = 5;
    int best = -1;
    float best_us = 0.f;
    for (size_t ci = 0; ci < cand.size() && rc == LIN_OK; ++ci) {
        const int vi = cand[ci];
        auto args = [&](int j) {
            return KArgs{W[j % count], S ? S[j % count] : nullptr, x, y,
                         (int)M, (int)N, (int)K, 1, nullptr, nullptr, x, 1e-6f};
        };
        // warm-up outside the capture (code load, LDS attribute)
        if ((rc = launch_variant(vi, args(0), ts)) != LIN_OK) break;
        if (hipStreamSynchronize(ts) != hipSuccess) { rc = LIN_ERR_HIP; break; }
        hipGraph_t g = nullptr;
        hipGraphExec_t ge = nullptr;
        if (hipStreamBeginCapture(ts, hipStreamCaptureModeThreadLocal) != hipSuccess) {
            rc = LIN_ERR_HIP;
            break;
        }
        int lrc = LIN_OK;
        for (int j = 0; j < n && lrc == LIN_OK; ++j) lrc = launch_variant(vi, args(j), ts);
        const hipError_t ce = hipStreamEndCapture(ts, &g);
        if (lrc != LIN_OK || ce != hipSuccess) rc = lrc != LIN_OK ? lrc : LIN_ERR_HIP;
        if (rc == LIN_OK && hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess)
            rc = LIN_ERR_HIP;
        float ms = 0.f;
        // warm replays; the first candidate gets more, since the first passes
        // over freshly allocated matrices run slower than the steady state
        const int warm = ci == 0 ? 16 : 1;
        for (int r = 0; r < warm && rc == LIN_OK; ++r)
            if (hipGraphLaunch(ge, ts) != hipSuccess) rc = LIN_ERR_HIP;
        if (rc == LIN_OK && hipEventRecord(e0, ts) != hipSuccess) rc = LIN_ERR_HIP;
        for (int r = 0; r < reps && rc == LIN_OK; ++r)
            if (hipGraphLaunch(ge, ts) != hipSuccess) rc = LIN_ERR_HIP;
        if (rc == LIN_OK && (hipEventRecord(e1, ts) != hipSuccess ||
                             hipEventSynchronize(e1) != hipSuccess ||
                             hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            rc = LIN_ERR_HIP;
        if (ge) (void)hipGraphExecDestroy(ge);
        if (g) (void)hipGraphDestroy(g);
        if (rc != LIN_OK) break;
        const float us = ms * 1000.f / (float)(reps * n);
        if (best < 0 || us < best_us) {
            best = vi;
            best_us = us;
        }
    }
    (void)hipStreamSynchronize(ts);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipStreamDestroy(ts);
    if (rc != LIN_OK) return rc;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        table()[Key(dev, kind, M, N, K)] = best;
    }
    if (out) {
        *out = registry()[best].cfg;
        out->us = best_us;
    }
    return LIN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free entry point

namespace lin {
namespace {

// Split-K scratch of lin_gemm_skinny_bf16_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends.  Layout as the library-owned
// workspace: kMaxTileCounters 32-bit tile counters, then the partial tiles.
constexpr size_t kStaticScratchBytes = LIN_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes > (size_t)kMaxTileCounters * 4, "room for the partial tiles");
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ void zero_words(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Per device: the array's device address (from hipGetSymbolAddress with that
// device current; host code never passes the array's name itself) and whether
// its tile counters have been cleared.  Fixed slots, so no host allocation.
constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::atomic<int> ready{0};
    void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address of the current device `dev`.  The first call on a
// device resolves it and clears the tile counters with a fill kernel on
// `stream` (stream-ordered before the caller's product; no memset node).
// Split-K kernels leave every counter they use at 0 again, so later calls
// find them cleared.
int device_scratch(int dev, hipStream_t stream, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return LIN_ERR_UNSUPPORTED;
    ScratchSlot& slot = g_scratch[dev];
    if (slot.ready.load(std::memory_order_acquire)) {
        *out = slot.ptr;
        return LIN_OK;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!slot.ready.load(std::memory_order_relaxed)) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LIN_ERR_HIP;
        hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, (uint32_t*)p,
                           kMaxTileCounters);
        if (hipGetLastError() != hipSuccess) return LIN_ERR_HIP;
        slot.ptr = p;
        slot.ready.store(1, std::memory_order_release);
    }
    *out = slot.ptr;
    return LIN_OK;
}

// The registry entry of `kind` matching cfg for this shape, found without
// building a candidate list.
int match_variant(int kind, int64_t M, int64_t N, int64_t K, const lin_config& cfg) {
    const auto& reg = registry();
    for (int i = 0; i < (int)reg.size(); ++i)
        if (same_cfg(reg[i].cfg, cfg) && applicable(reg[i], kind, M, N, K)) return i;
    return -1;
}

}  // namespace
}  // namespace lin

extern "C" int lin_gemm_skinny_bf16_noalloc(const void* W, const void* X, float* Y, int64_t M,
                                            int64_t N, int64_t K, const lin_config* cfg,
                                            void* stream) {
    const int kind = LIN_KIND_SKINNY_BF16;
    int st = check(kind, W, nullptr, X, Y, M, N, K);
    if (st != LIN_OK) return st > 0 ? LIN_OK : st;
    const int vi = cfg ? match_variant(kind, M, N, K, *cfg) : lookup(kind, M, N, K);
    if (vi < 0) return LIN_ERR_UNSUPPORTED;
    const size_t need = workspace_need(registry()[vi], M, N, K);
    void* ws = nullptr;
    if (need) {
        if (need > kStaticScratchBytes) return LIN_ERR_SCRATCH;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return LIN_ERR_HIP;
        if (int rc = device_scratch(dev, (hipStream_t)stream, &ws)) return rc;
    }
    KArgs a{W, nullptr, X, Y, (int)M, (int)N, (int)K, 1, nullptr};
    return launch_variant(vi, a, (hipStream_t)stream, nullptr, nullptr, nullptr, -1, ws);
}

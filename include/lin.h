/*
 * lin.h -- decode-step linear layers for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation.  A decode step multiplies every weight matrix of the model by
 * the current activation: y = W . x, each weight read from memory once and used
 * for one multiply-add (llm-rs benchmark post, section 2 "Decode with one request
 * is a memory problem"; yalm post, CPU matmul section: W (d,n) @ x (n,) with W
 * row-major).  A batch of M tokens reuses each weight M times, Y = X . W^T (llm-rs
 * benchmark post, section 3 "Batching moves decode from memory toward math").
 * Weights are bf16, or 4-bit integers with one fp16 scale per 64 weights along k
 * (tinyinfer post, TL;DR).
 *
 * Layouts (all row-major, contiguous, leading dimension = K):
 *   W   bf16    [N][K]     weights, N outputs by K inputs
 *   Wq  uint8   [N][K/2]   int4 codes, two per byte along k: byte j of a row holds
 *                          k = 2j in bits 0..3 and k = 2j+1 in bits 4..7; each
 *                          code is 4-bit two's complement q in [-8, 7]
 *   S   fp16    [N][K/64]  scale of each group of 64 consecutive k; w = q * s
 *   Wi  int8    [N][K]     INT8 weights q in [-127, 127] (lin_gemv_i8)
 *   Si  fp32    [N]        one scale per output channel (row); w = q * s
 *   x/X bf16    [M][K]     activations, one row per token
 *   y/Y fp32    [M][N]     outputs, overwritten (no accumulation into y)
 * Accumulation is fp32.  bf16 and INT8 weights: every product w x is exact in
 * fp32 and only the sums round, so every configuration is within
 * 1e-3 * sum_k |W[n][k] * x[m][k]| of the exact product, per output (the sums
 * contribute at most about (K / 2048 + 8) * 2^-24 of that term).
 * int4-g64 weights: the kernels multiply the exact bf16 codes 24 + q (no
 * conversion instruction per weight) and remove 24 * sum x per 16, 32 or 64
 * weights in fp32.  That removal adds rounding that is not proportional to
 * |q x|, so for int4 the guaranteed bound per output is
 *     |y - exact| <= 1e-4 * sum_k |W[n][k] x[m][k]|
 *                  + 4e-4 * sum_g s[n][g] * sum_{k in g} |x[m][k]|,
 * g over the row's scale groups.  It implies the 1e-3 * sum_k |W x| bound
 * whenever sum_k |q x| >= 0.45 * sum_k |x| over the row's groups (weighted by
 * their scales), i.e. the codes average at least about 0.45 in magnitude where
 * x is large: quantised Gaussian weights average about 2.  Rows dominated by
 * one outlier per group (most codes 0) typically stay far inside the 1e-3
 * bound as well, since the removal's roundings are random in sign; an input
 * built so that x vanishes exactly where a row's nonzero codes are can exceed
 * it, but never the bound above.
 *
 * Ownership and execution.  Every pointer is a device pointer owned by the
 * caller; the library never frees or retains them.  The compute entry points
 * (lin_gemv_bf16, lin_gemv_q4g64, lin_gemv_bf16_ep, lin_gemv_q4g64_ep,
 * lin_gemv_bf16_norm, lin_gemv_q4g64_norm, lin_gemv_i8, lin_gemv_i8_ep, lin_gemv_i8_norm,
 * lin_gemm_skinny_bf16,
 * lin_gemm_skinny_q4g64, lin_quantize_q4g64, lin_quantize_i8, lin_q4g64_tile)
 * validate their arguments in O(1), enqueue kernels on `stream` (a hipStream_t;
 * NULL = the null stream) and return without waiting: they never allocate,
 * never synchronise and are safe inside HIP graph capture.  Results are
 * deterministic: the same configuration on the same inputs gives the same bits.
 * Calls may be made from several host threads; the tuning table is guarded.
 * One exception to running calls concurrently: product calls whose
 * configuration splits K across workgroups (matrix-core configurations with
 * `split` > 1, chosen only by tuning or pinning) share their device's split-K
 * workspace, so two such calls must not overlap on different streams of one
 * device.  Every other call is reentrant.
 *
 * Errors.  Every entry point returns LIN_OK or a negative lin_status.  Argument
 * errors are detected before anything is enqueued, so nothing has run.
 * LIN_ERR_HIP means the HIP runtime reported an error (for example a launch
 * failure); the stream may then hold partial work.  No C++ exception crosses
 * this interface.  M == 0 or N == 0 is a valid empty call (nothing is enqueued;
 * pointers may be NULL).  K == 0 writes zeros to y (W and x may be NULL), except
 * for the RMSNorm products, which need K >= 1 (LIN_ERR_SHAPE).
 */
#ifndef LIN_H
#define LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lin_status {
    LIN_OK = 0,
    LIN_ERR_NULL = -1,        /* a required pointer is NULL */
    LIN_ERR_SHAPE = -2,       /* M, N or K out of range, or K not a multiple of 8 (bf16) / 64 (int4) / 16 (int8) */
    LIN_ERR_ALIGN = -3,       /* W, Wq, Wi, Wt, St, x or X not 16-byte aligned; y, Y, Si not 4-byte; S not 2-byte */
    LIN_ERR_UNSUPPORTED = -4, /* the requested configuration cannot run this shape */
    LIN_ERR_HIP = -5,         /* the HIP runtime reported an error */
    LIN_ERR_ARG = -6,         /* unknown kind, malformed configuration, bad index */
    LIN_ERR_SCRATCH = -7      /* lin_gemm_skinny_bf16_noalloc: the configuration needs more
                                 split-K scratch than LIN_STATIC_SCRATCH_BYTES */
} lin_status;

/* The products; `kind` selects one in the tuning calls. */
typedef enum lin_kind {
    LIN_KIND_GEMV_BF16 = 0,   /* lin_gemv_bf16 (and lin_gemv_bf16_ep) */
    LIN_KIND_GEMV_Q4G64 = 1,  /* lin_gemv_q4g64 (and lin_gemv_q4g64_ep) */
    LIN_KIND_SKINNY_BF16 = 2, /* lin_gemm_skinny_bf16 */
    LIN_KIND_SKINNY_Q4G64 = 3, /* lin_gemm_skinny_q4g64 (tiled int4-g64 weights) */
    LIN_KIND_GEMV_I8 = 4,      /* lin_gemv_i8 */
    LIN_KIND_GEMV_BF16_NORM = 5,  /* lin_gemv_bf16_norm (M == 1) */
    LIN_KIND_GEMV_Q4G64_NORM = 6, /* lin_gemv_q4g64_norm (M == 1) */
    LIN_KIND_GEMV_I8_NORM = 7     /* lin_gemv_i8_norm (M == 1) */
} lin_kind;

/* Kernel families. */
typedef enum lin_algo {
    LIN_ALGO_VALU = 1,        /* vector-ALU streaming product: each wavefront owns `rows` rows */
    LIN_ALGO_MFMA = 2         /* matrix-core tiles (the two skinny products) */
} lin_algo;

/* One launch configuration.  VALU: a wavefront owns `rows` consecutive rows and
 * streams them with 16-byte loads, `unroll` loads per lane and row in flight;
 * `split` wavefronts share a row group by splitting K and combine through LDS;
 * `stage_x` = 1 stages x in LDS once per workgroup; `tile_m` = tokens per
 * kernel instance.  MFMA: `rows` = W rows per workgroup, `tile_m` = tokens per
 * workgroup tile, `unroll` = k-blocks of 64 in flight per workgroup, `split` =
 * workgroups sharing one output tile by splitting K (their partial tiles go
 * through a library-owned workspace and are added in a fixed order, so results
 * stay deterministic); `stage_x` = 1: W streams through registers and a
 * 64-k block of X is staged in LDS per step; `stage_x` = 3 or 4: W and X
 * blocks both stream through an LDS ring of `unroll` stages filled by direct
 * global-to-LDS loads, in the matrix-core operand order (3) or in whole
 * 128-byte lines with a swizzled layout (4); `stage_x` = 5: the same line-order
 * ring with four more wavefronts per workgroup that issue every load, so the
 * product wavefronts never wait to issue one; `waves` = product wavefronts per
 * workgroup of the ring kernels (0 means the default, four; 8 puts two on each
 * SIMD).  LIN_KIND_SKINNY_Q4G64 has one family, `stage_x` = 4: codes, scales
 * and X stream through an LDS ring of `unroll` stages of 128 k, `rows` W rows
 * by `tile_m` tokens per workgroup, `split` as above.  `us` is filled by
 * lin_autotune (median microseconds per call, cold caches) and ignored on
 * input. */
typedef struct lin_config {
    int32_t algo;
    int32_t rows;
    int32_t unroll;
    int32_t split;
    int32_t stage_x;
    int32_t tile_m;
    int32_t waves;
    int32_t reserved;
    float us;
} lin_config;

/* Largest M accepted by lin_gemv_bf16 / lin_gemv_q4g64 / lin_gemv_i8, and by the skinny products. */
#define LIN_GEMV_MAX_M 8
#define LIN_SKINNY_MAX_M 256
/* Largest K accepted by every product. */
#define LIN_MAX_K (1 << 22)

/* y[m][n] = sum_k W[n][k] * x[m][k] for bf16 W [N][K], x [M][K]; fp32 y [M][N].
 * 1 <= M <= LIN_GEMV_MAX_M (the batch-1 decode GEMV is M = 1), K % 8 == 0. */
int lin_gemv_bf16(const void* W, const void* x, float* y,
                  int64_t M, int64_t N, int64_t K, void* stream);

/* The same product with int4-g64 weights: w[n][k] = q[n][k] * S[n][k/64].
 * K % 64 == 0, 1 <= M <= LIN_GEMV_MAX_M. */
int lin_gemv_q4g64(const void* Wq, const void* S, const void* x, float* y,
                   int64_t M, int64_t N, int64_t K, void* stream);

/* Epilogues fused into the batch-1 products (yalm post, GPU matmul section:
 * the residual add accumulated into the product's destination, and the gated
 * product silu(w1 x) * w3 x formed by the kernel that computes both products). */
typedef enum lin_epilogue {
    LIN_EPI_NONE = 0,    /* y = W x */
    LIN_EPI_ADD = 1,     /* y = W x + r; r fp32 [M][N], may be y itself (accumulate in place) */
    LIN_EPI_SWIGLU = 2   /* W has 2N rows, gate rows 0..N-1 then up rows N..2N-1 (as
                            concatenated at load); y[n] = silu(g_n) * u_n with g = W[0:N] x,
                            u = W[N:2N] x and silu(g) = g / (1 + exp(-g)); r unused */
} lin_epilogue;

/* lin_gemv_bf16 / lin_gemv_q4g64 (1 <= M <= LIN_GEMV_MAX_M) with a fused
 * epilogue, applied to every token row (r and y are [M][N]).  N counts
 * the outputs (the weight matrix has 2N rows for LIN_EPI_SWIGLU).  The
 * configuration is the one tuned or pinned for the plain product of the same
 * weight matrix, i.e. (kind, 1, 2N or N, K); with SWIGLU a wavefront keeps the
 * configuration's `rows` weight rows (rows/2 gate rows and the matching up
 * rows; one of each when rows is 1).  Error bound per output: for ADD,
 * 1e-3 * (sum_k |W x| + |r|); for SWIGLU, the GEMV bound propagated through
 * silu(g) u (1e-3 * (1.1 |u| sum_k |W_g x| + |silu(g)| sum_k |W_u x|)) plus a few
 * fp32 rounding steps of |y|.  M beyond LIN_GEMV_MAX_M returns LIN_ERR_SHAPE;
 * ADD with a NULL r LIN_ERR_NULL; an unknown epilogue LIN_ERR_ARG. */
int lin_gemv_bf16_ep(const void* W, const void* x, float* y,
                     int64_t M, int64_t N, int64_t K, int epilogue, const float* r, void* stream);
int lin_gemv_q4g64_ep(const void* Wq, const void* S, const void* x, float* y,
                      int64_t M, int64_t N, int64_t K, int epilogue, const float* r, void* stream);

/* lin_gemv_bf16_ep / lin_gemv_q4g64_ep with the RMSNorm of x folded into the
 * product as a prologue (tinyinfer post, decode section: the normalisation
 * moved into the projection kernels; TileInfer.jl post, "Incremental
 * acceleration": fused norms):
 *   h[k] = bf16(x[k] g[k] / sqrt(sum_k x[k]^2 / K + eps)),  y = W h (+ epilogue).
 * g: bf16 [K] gain, 16-byte aligned; eps >= 0 and finite (else LIN_ERR_ARG);
 * M == 1 and K >= 8 (bf16) or K >= 64 (int4-g64), else LIN_ERR_SHAPE; NULL g is
 * LIN_ERR_NULL.  x itself is not modified: each workgroup normalises its own
 * staged copy of x in LDS, next to a staged copy of g, before its first
 * product, so no normalised activation is written to memory.  Since every
 * workgroup repeats the prologue, these products are configurations of their
 * own kinds, LIN_KIND_GEMV_BF16_NORM and LIN_KIND_GEMV_Q4G64_NORM, tuned or
 * pinned for (kind, 1, 2N or N, K) like the plain products (the epilogue forms
 * share that configuration).  h is formed in fp32 (the sum of squares, then
 * x g times the reciprocal root) and rounded to bf16 to nearest-even; an entry
 * within a few fp32 steps of a bf16 rounding boundary may round the other way,
 * adding at most 2^-8 |W[n][k] h[k]| for that k to the bounds of the plain
 * product. */
int lin_gemv_bf16_norm(const void* W, const void* x, const void* g, float eps, float* y,
                       int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                       void* stream);
int lin_gemv_q4g64_norm(const void* Wq, const void* S, const void* x, const void* g, float eps,
                        float* y, int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                        void* stream);

/* The same product with INT8 weights and one fp32 scale per output channel
 * (TileInfer.jl post, "Pushing further with cheating: INT8 quantization": the
 * INT8 values are multiplied in and the channel's scale applied once at the
 * end): y[m][n] = Si[n] * sum_k Wi[n][k] * x[m][k].  K % 16 == 0,
 * 1 <= M <= LIN_GEMV_MAX_M; Wi 16-byte and Si 4-byte aligned. */
int lin_gemv_i8(const void* Wi, const void* Si, const void* x, float* y,
                int64_t M, int64_t N, int64_t K, void* stream);

/* lin_gemv_i8 with a fused epilogue (as lin_gemv_bf16_ep; the gated
 * product applies each row's scale before the gate: silu(Si[n] g_n) Si[N+n] u_n,
 * with Si holding the 2N scales of the gate|up rows), and with the RMSNorm
 * prologue as well (as lin_gemv_bf16_norm; kind LIN_KIND_GEMV_I8_NORM, K >= 16).
 * Same argument rules and bounds as those entry points. */
int lin_gemv_i8_ep(const void* Wi, const void* Si, const void* x, float* y,
                   int64_t M, int64_t N, int64_t K, int epilogue, const float* r, void* stream);
int lin_gemv_i8_norm(const void* Wi, const void* Si, const void* x, const void* g, float eps,
                     float* y, int64_t M, int64_t N, int64_t K, int epilogue, const float* r,
                     void* stream);

/* Batched-token product Y = X . W^T for 1 <= M <= LIN_SKINNY_MAX_M tokens,
 * K % 8 == 0.  Small M streams W once through the vector ALUs; larger M runs on
 * the matrix cores; the crossover is part of the tuned configuration. */
int lin_gemm_skinny_bf16(const void* W, const void* X, float* Y,
                         int64_t M, int64_t N, int64_t K, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the product of
 * lin_gemm_skinny_bf16, in configuration *cfg (one of the candidates of
 * (LIN_KIND_SKINNY_BF16, M, N, K); NULL: the configuration lin_get_config
 * reports), where a split-K configuration keeps its partial tiles and tile
 * counters in a static device array of LIN_STATIC_SCRATCH_BYTES instead of the
 * library's workspace, so it needs no earlier lin_set_config or lin_autotune
 * to reserve one.  Allocates no device memory and never synchronises.  The
 * array is part of the library's code object: each GPU the library runs on
 * holds one copy until the process ends.  The first call on a device looks up
 * the array's address and clears its tile counters with a small kernel on
 * `stream`; split-K kernels leave the counters cleared.  Every call on a GPU
 * shares that GPU's array: calls whose configurations use split-K must not
 * overlap on one GPU (different streams or host threads race on it).  A
 * configuration needing more than the array returns LIN_ERR_SCRATCH, an
 * unknown one LIN_ERR_UNSUPPORTED; the other argument rules are those of
 * lin_gemm_skinny_bf16. */
#define LIN_STATIC_SCRATCH_BYTES (16u << 20)
int lin_gemm_skinny_bf16_noalloc(const void* W, const void* X, float* Y,
                                 int64_t M, int64_t N, int64_t K, const lin_config* cfg,
                                 void* stream);

/* Batched-token product with int4-g64 weights, for 1 <= M <= LIN_SKINNY_MAX_M
 * tokens: Y[m][n] = sum_k q[n][k] * S[n][k/64] * X[m][k], fp32 Y [M][N], bf16 X
 * [M][K], K % 64 == 0, the weights in the tiled layout of lin_q4g64_tile (Wt
 * and St 16-byte aligned).  The reordering is the one the llm-rs benchmark
 * post (section 6) describes for 4-bit GEMMs: done once at load time, so that
 * one 16-byte load gives each lane exactly the codes of its matrix-core
 * operands.  Runs on the matrix cores for every M; products are exact in fp32
 * and the scales are applied in fp32 per group (the bound above holds). */
int lin_gemm_skinny_q4g64(const void* Wt, const void* St, const void* X, float* Y,
                          int64_t M, int64_t N, int64_t K, void* stream);

/* Bytes of the tiled int4-g64 layout of an N x K matrix (K % 64 == 0):
 * *wt_bytes = ceil(N/16) * ceil(K/128) * 1024, *st_bytes = ceil(N/16) *
 * ceil(K/128) * 64. */
int lin_q4g64_tiled_size(int64_t N, int64_t K, int64_t* wt_bytes, int64_t* st_bytes);

/* Load-time weight preparation for lin_gemm_skinny_q4g64: rearrange Wq [N][K/2]
 * and S [N][K/64] (the layouts above; Wq 16-byte, S 2-byte aligned) into
 * caller-owned Wt and St (16-byte aligned, sizes from lin_q4g64_tiled_size).
 * With N16 = ceil(N/16) and KB = ceil(K/128):
 *   Wt: N16 x KB units of 1024 bytes, unit (T, j) at byte (T * KB + j) * 1024;
 *       its dword 4 l + t (lane l < 64, t < 4) holds the 8 codes of Wq row
 *       16 T + (l mod 16) at k = k0 + e, e < 8, k0 = 128 j + 32 t + 8 (l / 16)
 *       (Wq bytes 64 j + 16 t + 4 (l / 16) .. + 3), reordered: the code of
 *       k0 + 2 i in bits 4 i .. 4 i + 3 and that of k0 + 2 i + 1 in bits
 *       16 + 4 i .. 19 + 4 i (i < 4);
 *   St: KB x N16 units of 64 bytes, unit (j, T) at byte (j * N16 + T) * 64;
 *       its fp16 element 2 r + h (r < 16, h < 2) is S[16 T + r][2 j + h].
 * Entries past row N - 1 or past k = K - 1 are zero.  Enqueued on `stream`;
 * allocates nothing.  N == 0 or K == 0 enqueues nothing. */
int lin_q4g64_tile(const void* Wq, const void* S, void* Wt, void* St,
                   int64_t N, int64_t K, void* stream);

/* Load-time tuning (tinyinfer post, "v0.2": time the candidates on every
 * distinct shape when the model loads, keep the fastest).  Times every
 * candidate configuration of `kind` for (M, N, K) on the caller's buffers,
 * which must be valid for that kind (S is used only by the int4 and INT8 kinds
 * and may be NULL otherwise; W and S are Wt and St for LIN_KIND_SKINNY_Q4G64, Wi
 * and Si for LIN_KIND_GEMV_I8 and LIN_KIND_GEMV_I8_NORM; for the RMSNorm kinds M must be 1 and x also
 * stands in for the gain; y receives scratch results).  Each timed call starts
 * from cold caches.  The fastest configuration is stored in the per-device
 * table and used by later calls with the same (kind, M, N, K); if `out` is not
 * NULL it receives it, with `us` set.  Unlike the compute calls this one
 * allocates a cache-flush buffer on first use and the split-K workspace the
 * candidates need (both kept until process exit), synchronises `stream` and
 * must not be called during graph capture. */
int lin_autotune(int kind, const void* W, const void* S, const void* x, float* y,
                 int64_t M, int64_t N, int64_t K, void* stream, lin_config* out);

/* The same load-time tuning timed the way a decode step runs the layer: every
 * candidate is captured as one graph of back-to-back calls cycling over the
 * `count` >= 1 weight matrices W[0..count-1] (and S[0..count-1] for the
 * int4 and INT8 kinds; S may be NULL otherwise) of the same shape, e.g. the
 * layers of a model, and the graph is replayed; `us` is the mean time per
 * call.  W and S are host arrays of device pointers, owned by the caller and
 * only read during the call.  Stores the fastest configuration like
 * lin_autotune and has the same allocation, synchronisation and
 * no-capture rules; it runs the candidates on a stream of its own. */
int lin_autotune_set(int kind, const void* const* W, const void* const* S, int count,
                     const void* x, float* y, int64_t M, int64_t N, int64_t K, void* stream,
                     lin_config* out);

/* Candidate configurations for (kind, M, N, K), in a fixed order: returns how
 * many there are (>= 0) or a negative status.  lin_candidate writes number
 * `index` to *out. */
int lin_num_candidates(int kind, int64_t M, int64_t N, int64_t K);
int lin_candidate(int kind, int64_t M, int64_t N, int64_t K, int index, lin_config* out);

/* The configuration the next call of (kind, M, N, K) on the current device will
 * use: the tuned or pinned entry if there is one, else the built-in default. */
int lin_get_config(int kind, int64_t M, int64_t N, int64_t K, lin_config* out);

/* Pin `cfg` for (kind, M, N, K) on the current device (it must be one of the
 * candidates), or remove the entry when cfg is NULL.  A load-time call: a
 * split-K configuration makes the library grow its per-device workspace here
 * (allocation and device synchronisation), never in the product calls; a
 * product call whose pinned configuration lacks workspace returns
 * LIN_ERR_UNSUPPORTED.  A configuration that stages x in more than 64 KB of
 * LDS has that limit raised for its kernel here as well (otherwise on its
 * first launch).  Product calls that use split-K share the device's
 * workspace, so such calls on one device must not run concurrently on
 * different streams.  The library never frees a workspace (a grown one keeps
 * the old buffer allocated until the process ends), so a graph captured with a
 * split-K configuration stays valid after later calls grow the workspace. */
int lin_set_config(int kind, int64_t M, int64_t N, int64_t K, const lin_config* cfg);

/* Load-time weight preparation: quantise bf16 W [N][K] (K % 64 == 0) to the
 * int4-g64 layout above.  Per row and group of 64 k: a = max |w|;
 * s = fp16 nearest to a/7 (ties to even; saturates at 65504);
 * q = s > 0 ? clamp(round_half_even(w / s), -8, 7) : 0, with w/s in fp64.
 * Writes Wq [N][K/2] and S [N][K/64].  W must hold finite values. */
int lin_quantize_q4g64(const void* W, void* Wq, void* S, int64_t N, int64_t K, void* stream);

/* Load-time weight preparation for lin_gemv_i8: quantise bf16 W [N][K]
 * (K % 16 == 0) to INT8 with one fp32 scale per row (TileInfer.jl post, INT8
 * section: scale = max |w| / 127, each weight rounded to the nearest multiple of
 * the scale).  Per row: a = max_k |w|; s = fp32 nearest to a/127 (the quotient
 * formed in fp64, rounded once); q = s > 0 ? clamp(round_half_even(w / s),
 * -127, 127) : 0 with w / s in fp64.  Writes Wi [N][K] and Si [N].  W must hold
 * finite values. */
int lin_quantize_i8(const void* W, void* Wi, void* Si, int64_t N, int64_t K, void* stream);

/* Measurement: read every byte of `buf` (device, 16-byte aligned, `bytes` a
 * multiple of 16) once and discard it.  This is the ceiling a product is
 * measured against (llm-rs design post, section 6: track the share of a
 * ceiling): the same bytes, streamed by a kernel that does nothing else, with
 * the launch shape the products use at their best (short wavefronts of four
 * 16-byte loads per lane).  Enqueued on `stream`; allocates nothing. */
int lin_stream_read(const void* buf, int64_t bytes, void* stream);

/* Static description of a status code. */
const char* lin_status_string(int status);

/* Interface version: (major << 16) | minor. */
int lin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIN_H */

// Kernel variants known to the host library.  Each kernel source file appends
// its instantiations to the registry; the C-ABI layer picks one per call.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/lin.h"
#include "kern_common.h"

namespace lin {

struct Variant {
    int kind;          // LIN_KIND_*
    lin_config cfg;    // public description (algo, rows, unroll, split, stage_x, tile_m, waves)
    int mt;            // VALU: tokens per instance (M <= mt); MFMA: 0 (any M in range)
    int min_m;         // smallest M this variant accepts
    const void* func;  // __global__ function
    // Workgroups and dynamic LDS bytes for a shape; returns false if the shape
    // does not fit this variant (for example LDS too small for K).
    bool (*geometry)(const Variant&, int M, int N, int K, dim3* grid, size_t* lds);
    // Split-K workspace bytes this variant needs for a shape (0: none).
    size_t (*workspace)(const Variant&, int M, int N, int K);
    int block = 0;     // threads per workgroup (0: kBlock)
    // The same configuration with a fused epilogue (index kEpiAdd, kEpiSwiglu;
    // batch-1 GEMV variants only), or nullptr.
    // For the RMSNorm kinds, func is the prologue kernel without an epilogue
    // and epi[] the prologue kernels with one.
    const void* epi[3] = {nullptr, nullptr, nullptr};
};

void register_gemv_bf16(std::vector<Variant>& out);
void register_gemv_q4g64(std::vector<Variant>& out);
void register_gemm_mfma(std::vector<Variant>& out);
void register_gemm_mfma_ring(std::vector<Variant>& out);
void register_gemm_q4_ring(std::vector<Variant>& out);
void register_gemv_i8(std::vector<Variant>& out);
void register_gemv_q4t(std::vector<Variant>& out);
void register_gemv_q4x(std::vector<Variant>& out);

// Quantiser launches (int4-g64 and INT8 weight preparation).
hipError_t launch_quantize_q4g64(const void* W, void* Wq, void* S, int N, int K, hipStream_t stream);
hipError_t launch_quantize_i8(const void* W, void* Wq, void* S, int N, int K, hipStream_t stream);

// Matrix-core tiled int4-g64 layout: sizes and the rearrangement launch.
void q4g64_tiled_bytes(int64_t N, int64_t K, int64_t* wt, int64_t* st);
hipError_t launch_tile_q4g64(const void* Wq, const void* S, void* Wt, void* St, int N, int K,
                             hipStream_t stream);

// Cache sweep used while tuning: reads n 16-byte words.
hipError_t launch_flush(void* buf, size_t n16, uint32_t salt, hipStream_t stream);

// Read-only streaming pass (achievable-bandwidth ceiling).
hipError_t launch_stream_read(const void* buf, size_t bytes, hipStream_t stream);

// Largest dynamic LDS a workgroup may ask for (gfx950: 160 KB per compute
// unit; a little is left for the kernels' static arrays).
constexpr size_t kMaxDynLds = 156 * 1024;

}  // namespace lin
